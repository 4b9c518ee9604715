// RWKV-4 WKV kernels for gfx950: recurrent step, state init, and the
// time-parallel forward as a single-pass tiled scan.
//
// What is computed: [RWKV-digest] "RWKV - Reinventing RNNs for the
// Transformer Era" (paper digest), Method > (2) Time-mixing (WKV): WKV_t and
// its recurrent form a_t = e^{-w} a_{t-1} + e^{k_t} v_t (same for b with 1),
// WKV_t = (a_{t-1} + e^{u+k_t} v_t) / (b_{t-1} + e^{u+k_t}).  The time-parallel
// form rests on the associativity of "decay then add" (same page, atomic
// insight on the training/inference duality).
//
// Forward design (one launch, 12 bytes of HBM traffic per element):
//   * a workgroup owns one 64-channel block of one sequence and a tile of
//     L*NW tokens; each of its NW waves holds L tokens of k and v for its 64
//     channels in registers (one lane per channel, loads coalesced along c);
//   * each wave summarises its L tokens from an empty history; wave 0 joins
//     the NW summaries into the tile aggregate and publishes it;
//   * wave 0 then walks back over earlier tiles of the same channel block
//     (decoupled look-back): an earlier tile's inclusive history ends the
//     walk, its aggregate is folded in and the walk continues;
//   * every wave rebuilds its own starting history from the tile prefix and
//     the summaries of the waves before it, then rescans its tokens from
//     registers and writes y.
// Workgroups take tiles in ticket order, so every tile a workgroup waits on
// belongs to a workgroup that is already running: the waits always end.
#include "wkv_device.h"
#include "wkv_internal.h"

#include <stdlib.h>
#include <stdio.h>

namespace rwkv {

namespace {

// Header words (uint32) at the start of the forward workspace.
enum : int { kHdrTicket = 0, kHdrDone = 1, kHdrEpoch = 2, kHdrError = 3 };
// Look-back polls before a workgroup gives up (about seconds); then it
// raises the error word and writes NaN so that no wait can last forever.
constexpr uint32_t kSpinLimit = 1u << 24;

__device__ __forceinline__ uint32_t hdr_load(uint32_t* h, int i) {
  return __hip_atomic_load(h + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void hdr_store(uint32_t* h, int i, uint32_t x) {
  __hip_atomic_store(h + i, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t hdr_add(uint32_t* h, int i, uint32_t x) {
  return __hip_atomic_fetch_add(h + i, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void publish(uint64_t* slot, const Hist& h, uint32_t tag) {
  tagged_store(slot + 0 * 64, h.A, tag);
  tagged_store(slot + 1 * 64, h.Bd, tag);
  tagged_store(slot + 2 * 64, h.kr, tag);
  tagged_store(slot + 3 * 64, h.n, tag);
}

// History of `n` tokens (n <= L) from an empty start, evaluated after the
// last one, by a fixed reference instead of a running maximum: token s has
// log2-weight m_s = k2_s - (n-1-s) w2; with P = max_s m_s every term is
// 2^(m_s - P) <= 1 and the largest is exactly 1, so nothing overflows and the
// sum never underflows to 0.  Costs one exp2 per token and no selects.
template <int L>
__device__ __forceinline__ Hist summarize(const float (&kk)[L], const float (&vv)[L], int n,
                                          float w2) {
  // Decay steps from token s to the evaluation point (padding: none, and the
  // padding exponent is pushed far below the maximum).
  auto expo = [&](int s) {
    const bool full = n == L;
    const float back = full ? float(L - 1 - s) : float(n - 1 - s);
    const float m = fmaf(-back, w2, kk[s]);
    return (full || s < n) ? m : kEmptyP;
  };
  float P = kEmptyP;
#pragma unroll
  for (int s = 0; s < L; ++s) P = fmaxf(P, expo(s));
  float A = 0.f, Bd = 0.f;
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const float e = exp2_fast(expo(s) - P);  // exactly 0 for the padding tokens
    A = fmaf(e, vv[s], A);
    Bd += e;
  }
  return n > 0 ? Hist{A, Bd, P, 0.f} : hist_empty();
}

template <int L, int NW>
__global__ __launch_bounds__(64 * NW) void wkv4_fwd_tiled(
    int T, int C, int n_cblk, int groups, int n_tiles,
    const float* __restrict__ w, const float* __restrict__ u,
    const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ y,
    uint32_t* __restrict__ hdr, uint64_t* __restrict__ slots) {
  constexpr int TILE = L * NW;
  constexpr int SLOT = kWkv4SlotWords * 64;  // words per (tile, channel block)
  __shared__ int s_ticket;
  __shared__ uint32_t s_tag;
  __shared__ float s_sum[NW][4][64];
  __shared__ float s_pre[4][64];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t total = uint32_t(n_tiles) * uint32_t(groups);
  if (threadIdx.x == 0) {
    s_tag = hdr_load(hdr, kHdrEpoch) + 1u;
    s_ticket = int(hdr_add(hdr, kHdrTicket, 1u));
  }
  __syncthreads();
  const int ticket = __builtin_amdgcn_readfirstlane(s_ticket);
  const uint32_t tag = __builtin_amdgcn_readfirstlane(s_tag);
  // A workspace that was not zero-filled can hand out tickets past the grid;
  // flag it and touch nothing.
  if (uint32_t(ticket) >= total) {
    if (threadIdx.x == 0)
      __hip_atomic_fetch_or(hdr + kHdrError, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int tile = ticket / groups;
  const int g = ticket - tile * groups;
  const int bi = g / n_cblk;
  const int cb = g - bi * n_cblk;
  const int c = cb * 64 + lane;
  const bool valid = c < C;
  const int cc = valid ? c : C - 1;  // parameter reads stay in bounds
  const float w2 = w[cc] * kLog2e;
  const float u2 = u[cc] * kLog2e;

  const int tile_t0 = tile * TILE;
  const int t0 = tile_t0 + wid * L;
  const int n = max(0, min(L, T - t0));
  // Wave-uniform row base; the lane adds only its channel.
  const size_t row0 = (size_t(bi) * size_t(T) + size_t(t0)) * size_t(C) + size_t(cb) * 64;
  const float* kp = k + row0;
  const float* vp = v + row0;
  const int lc = valid ? lane : (C - 1) - cb * 64;

  float kk[L], vv[L];
  if (n == L) {
#pragma unroll
    for (int s = 0; s < L; ++s) {
      kk[s] = kp[size_t(s) * C + lc];
      vv[s] = vp[size_t(s) * C + lc];
    }
  } else {
#pragma unroll
    for (int s = 0; s < L; ++s) {
      kk[s] = s < n ? kp[size_t(s) * C + lc] : 0.f;
      vv[s] = s < n ? vp[size_t(s) * C + lc] : 0.f;
    }
  }
#pragma unroll
  for (int s = 0; s < L; ++s) kk[s] *= kLog2e;

  // Pass 1: this wave's tokens from an empty history.
  {
    const Hist h = summarize<L>(kk, vv, n, w2);
    s_sum[wid][0][lane] = h.A;
    s_sum[wid][1][lane] = h.Bd;
    s_sum[wid][2][lane] = h.kr;
    s_sum[wid][3][lane] = h.n;
  }
  __syncthreads();

  // Tile prefix: wave 0 publishes the aggregate and looks back.
  if (wid == 0) {
    Hist agg = Hist{s_sum[0][0][lane], s_sum[0][1][lane], s_sum[0][2][lane], s_sum[0][3][lane]};
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      const int ni = max(0, min(L, T - (tile_t0 + i * L)));
      agg = hist_concat(agg, Hist{s_sum[i][0][lane], s_sum[i][1][lane], s_sum[i][2][lane],
                                  s_sum[i][3][lane]},
                        float(ni), w2);
    }
    const int tile_n = min(TILE, T - tile_t0);
    uint64_t* mine = slots + (size_t(tile) * groups + g) * SLOT + lane;
    Hist pre = hist_empty();
    if (tile == 0) {
      publish(mine + 4 * 64, agg, tag);
    } else {
      publish(mine, agg, tag);
      Hist acc = hist_empty();  // tiles (pos, tile) folded so far
      float acc_n = 0.f;
      int pos = tile - 1;
      uint32_t spins = 0;
      while (true) {
        const uint64_t* sp = slots + (size_t(pos) * groups + g) * SLOT + lane;
        // One lane polls the first word of each history; the whole wave
        // reads the payload only once it is there.  0: nothing yet,
        // 1: aggregate, 2: inclusive.
        int state = 0;
        if (lane == 0) {
          const uint64_t iw = tagged_load(sp + 4 * 64);
          const uint64_t aw = tagged_load(sp);
          state = tag_ok(iw, tag) ? 2 : ((pos > 0 && tag_ok(aw, tag)) ? 1 : 0);
        }
        state = __builtin_amdgcn_readfirstlane(__shfl(state, 0));
        if (state != 0) {
          const uint64_t* q = sp + (state == 2 ? 4 * 64 : 0);
          const uint64_t x0 = tagged_load(q);
          const uint64_t x1 = tagged_load(q + 64);
          const uint64_t x2 = tagged_load(q + 128);
          const uint64_t x3 = tagged_load(q + 192);
          if (__all(tag_ok(x0, tag) && tag_ok(x1, tag) && tag_ok(x2, tag) && tag_ok(x3, tag))) {
            const Hist hx = Hist{tag_val(x0), tag_val(x1), tag_val(x2), tag_val(x3)};
            acc = hist_concat(hx, acc, acc_n, w2);
            if (state == 2) {
              pre = acc;
              break;
            }
            acc_n += float(TILE);
            --pos;
            continue;
          }
        }
        if (++spins > kSpinLimit) {
          if (lane == 0)
            __hip_atomic_fetch_or(hdr + kHdrError, 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
          const float nan = __builtin_nanf("");
          pre = Hist{nan, nan, nan, 0.f};
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      publish(mine + 4 * 64, hist_concat(pre, agg, float(tile_n), w2), tag);
    }
    s_pre[0][lane] = pre.A;
    s_pre[1][lane] = pre.Bd;
    s_pre[2][lane] = pre.kr;
    s_pre[3][lane] = pre.n;
  }
  __syncthreads();

  // Pass 2: start from the tile prefix plus the earlier waves, emit y.
  if (n > 0) {
    Hist hs = Hist{s_pre[0][lane], s_pre[1][lane], s_pre[2][lane], s_pre[3][lane]};
    for (int i = 0; i < wid; ++i)
      hs = hist_concat(hs, Hist{s_sum[i][0][lane], s_sum[i][1][lane], s_sum[i][2][lane],
                                s_sum[i][3][lane]},
                       float(L), w2);
    float* yp = y + row0;
    if (n == L) {
#pragma unroll
      for (int s = 0; s < L; ++s) {
        const float ys = hist_read_push(hs, kk[s], vv[s], u2, w2);
        if (valid) yp[size_t(s) * C + lane] = ys;
      }
    } else {
#pragma unroll
      for (int s = 0; s < L; ++s) {
        if (s < n) {
          const float ys = hist_read_push(hs, kk[s], vv[s], u2, w2);
          if (valid) yp[size_t(s) * C + lane] = ys;
        }
      }
    }
  }

  // The last workgroup to finish resets the counters for the next call.
  if (threadIdx.x == 0) {
    const uint32_t d = hdr_add(hdr, kHdrDone, 1u);
    if (d == total - 1u) {
      hdr_store(hdr, kHdrTicket, 0u);
      hdr_store(hdr, kHdrDone, 0u);
      hdr_store(hdr, kHdrEpoch, tag);
    }
  }
}

// One thread per 4 consecutive channels of one stream: the step is
// elementwise, 36 bytes of traffic per element.
__device__ __forceinline__ void step_one(float& a, float& b, float& p, float w, float u,
                                         float k, float v, float& y) {
  const float w2 = w * kLog2e;
  Hist h{a, b, p * kLog2e, 0.f};
  y = hist_read_push(h, k * kLog2e, v, u * kLog2e, w2);
  a = h.A;
  b = h.Bd;
  p = hist_p(h, w2) * kLn2;
}

__global__ __launch_bounds__(256) void wkv4_step_vec4(
    int B, int C4, float4* __restrict__ a, float4* __restrict__ b, float4* __restrict__ p,
    const float4* __restrict__ w, const float4* __restrict__ u,
    const float4* __restrict__ k, const float4* __restrict__ v, float4* __restrict__ y) {
  const int c4 = blockIdx.x * 256 + threadIdx.x;
  if (c4 >= C4) return;
  const float4 wv = w[c4], uv = u[c4];
  for (int row = blockIdx.y; row < B; row += gridDim.y) {
    const size_t i = size_t(row) * C4 + c4;
    float4 av = a[i], bv = b[i], pv = p[i];
    const float4 kv = k[i], vv = v[i];
    float4 yv;
    step_one(av.x, bv.x, pv.x, wv.x, uv.x, kv.x, vv.x, yv.x);
    step_one(av.y, bv.y, pv.y, wv.y, uv.y, kv.y, vv.y, yv.y);
    step_one(av.z, bv.z, pv.z, wv.z, uv.z, kv.z, vv.z, yv.z);
    step_one(av.w, bv.w, pv.w, wv.w, uv.w, kv.w, vv.w, yv.w);
    a[i] = av;
    b[i] = bv;
    p[i] = pv;
    y[i] = yv;
  }
}

__global__ __launch_bounds__(256) void wkv4_step_scalar(
    int B, int C, float* __restrict__ a, float* __restrict__ b, float* __restrict__ p,
    const float* __restrict__ w, const float* __restrict__ u,
    const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ y) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const float wc = w[c], uc = u[c];
  for (int row = blockIdx.y; row < B; row += gridDim.y) {
    const size_t i = size_t(row) * C + c;
    float av = a[i], bv = b[i], pv = p[i], yv;
    step_one(av, bv, pv, wc, uc, k[i], v[i], yv);
    a[i] = av;
    b[i] = bv;
    p[i] = pv;
    y[i] = yv;
  }
}

__global__ __launch_bounds__(256) void wkv4_state_fill(size_t n, float* __restrict__ a,
                                                       float* __restrict__ b,
                                                       float* __restrict__ p) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256) {
    a[i] = 0.f;
    b[i] = 0.f;
    p[i] = kEmptyP;
  }
}

struct Variant {
  int L, NW;
};
// Instantiated tile shapes (tokens per wave, waves per workgroup).
constexpr Variant kVariants[] = {{64, 4}, {64, 1}, {32, 4}, {32, 8}, {16, 4}, {64, 2}, {16, 1}};

template <int L, int NW>
hipError_t launch_tiled(const Wkv4Plan& pl, int64_t T, int64_t C, const float* w,
                        const float* u, const float* k, const float* v, float* y, void* ws,
                        hipStream_t stream) {
  uint32_t* hdr = static_cast<uint32_t*>(ws);
  uint64_t* slots = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + kWkv4HeaderBytes);
  const unsigned grid = unsigned(pl.n_tiles * pl.groups);
  hipLaunchKernelGGL((wkv4_fwd_tiled<L, NW>), dim3(grid), dim3(64 * NW), 0, stream, int(T),
                     int(C), int(pl.n_cblk), int(pl.groups), int(pl.n_tiles), w, u, k, v, y,
                     hdr, slots);
  return hipGetLastError();
}

}  // namespace

bool wkv4_plan(int64_t B, int64_t T, int64_t C, Wkv4Plan* plan) {
  // 32 tokens per wave keeps k, v and the history in about 100 VGPRs
  // (4 waves per SIMD); 8 waves stack a 256-token tile.
  int L = 32, NW = 8;
  if (T <= 64) {
    L = 64;
    NW = 1;
  }
  if (const char* env = getenv("RWKV_WKV4_TILE")) {
    int l = 0, nw = 0;
    if (sscanf(env, "%d,%d", &l, &nw) == 2) {
      for (const Variant& vv : kVariants)
        if (vv.L == l && vv.NW == nw) {
          L = l;
          NW = nw;
        }
    }
  }
  Wkv4Plan p;
  p.L = L;
  p.NW = NW;
  p.tile = int64_t(L) * NW;
  p.n_tiles = (T + p.tile - 1) / p.tile;
  p.n_cblk = (C + 63) / 64;
  p.groups = B * p.n_cblk;
  // Tickets, token indices and channel indices are 32-bit in the kernel.
  if (p.n_tiles * p.groups >= (int64_t(1) << 31) || T >= (int64_t(1) << 31) ||
      C >= (int64_t(1) << 31) || p.groups >= (int64_t(1) << 31))
    return false;
  p.ws_bytes = kWkv4HeaderBytes +
               size_t(p.n_tiles) * size_t(p.groups) * kWkv4SlotWords * 64 * sizeof(uint64_t);
  *plan = p;
  return true;
}

hipError_t wkv4_forward_launch(const Wkv4Plan& pl, int64_t B, int64_t T, int64_t C,
                               const float* w, const float* u, const float* k,
                               const float* v, float* y, void* ws, hipStream_t stream) {
  (void)B;
  switch (pl.L * 100 + pl.NW) {
    case 6404: return launch_tiled<64, 4>(pl, T, C, w, u, k, v, y, ws, stream);
    case 6401: return launch_tiled<64, 1>(pl, T, C, w, u, k, v, y, ws, stream);
    case 3204: return launch_tiled<32, 4>(pl, T, C, w, u, k, v, y, ws, stream);
    case 3208: return launch_tiled<32, 8>(pl, T, C, w, u, k, v, y, ws, stream);
    case 1604: return launch_tiled<16, 4>(pl, T, C, w, u, k, v, y, ws, stream);
    case 6402: return launch_tiled<64, 2>(pl, T, C, w, u, k, v, y, ws, stream);
    case 1601: return launch_tiled<16, 1>(pl, T, C, w, u, k, v, y, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t wkv4_state_init_launch(int64_t B, int64_t C, float* a, float* b, float* p,
                                  hipStream_t stream) {
  const size_t n = size_t(B) * size_t(C);
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(wkv4_state_fill, dim3(unsigned(blocks)), dim3(256), 0, stream, n, a, b, p);
  return hipGetLastError();
}

hipError_t wkv4_step_launch(int64_t B, int64_t C, float* a, float* b, float* p,
                            const float* w, const float* u, const float* k, const float* v,
                            float* y, hipStream_t stream) {
  const unsigned rows = unsigned(B < 65535 ? B : 65535);
  if (C % 4 == 0) {
    const int64_t C4 = C / 4;
    const dim3 grid(unsigned((C4 + 255) / 256), rows);
    hipLaunchKernelGGL(wkv4_step_vec4, grid, dim3(256), 0, stream, int(B), int(C4),
                       reinterpret_cast<float4*>(a), reinterpret_cast<float4*>(b),
                       reinterpret_cast<float4*>(p), reinterpret_cast<const float4*>(w),
                       reinterpret_cast<const float4*>(u), reinterpret_cast<const float4*>(k),
                       reinterpret_cast<const float4*>(v), reinterpret_cast<float4*>(y));
  } else {
    const dim3 grid(unsigned((C + 255) / 256), rows);
    hipLaunchKernelGGL(wkv4_step_scalar, grid, dim3(256), 0, stream, int(B), int(C), a, b, p,
                       w, u, k, v, y);
  }
  return hipGetLastError();
}

}  // namespace rwkv
