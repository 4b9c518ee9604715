// Building blocks shared by the RWKV-4 forward and backward scans on gfx950:
// the per-call tag and tile claim, workspace header words, buffer-resource
// streaming of [B, T, C] rows, the fixed-reference summary of a wave's
// tokens, and shared-memory slots for per-channel histories.
#pragma once

#include "wkv_device.h"
#include "wkv_internal.h"

namespace rwkv {
namespace scan {

// Look-back polls without progress before a workgroup gives up (seconds);
// it then raises the error word and writes NaN, so no wait lasts forever.
constexpr uint32_t kSpinLimit = 1u << 24;  // default; the kernels take theirs as an argument
// Earlier tiles polled per round trip by the look-back.
constexpr int kWin = 16;

__device__ __forceinline__ void raise_error(uint32_t* err, uint32_t bit) {
  __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Header words (uint32) at the start of a scan workspace.
enum : int { kHdrError = 0, kHdrEpoch = 1, kHdrClaimed = 2 };
// Bits of the error word (sticky until the workspace is zero-filled again).
constexpr uint32_t kErrGaveUp = 1u;     // a look-back exceeded its spin limit
constexpr uint32_t kErrNotZeroed = 2u;  // a claim found a workspace never zero-filled

__device__ __forceinline__ uint32_t hdr_load(uint32_t* h, int i) {
  return __hip_atomic_load(h + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void hdr_store(uint32_t* h, int i, uint32_t x) {
  __hip_atomic_store(h + i, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t hdr_add(uint32_t* h, int i, uint32_t x) {
  return __hip_atomic_fetch_add(h + i, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A workgroup barrier for data exchanged through shared memory only.
// __syncthreads also fences global memory, which on gfx9 waits for every
// outstanding load and store of the wave (s_waitcnt vmcnt(0)), including row
// loads meant to stay in flight and stores nobody in the workgroup reads.
// Here only this wave's shared-memory operations complete first; the empty
// asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// k, v and y stream through buffer resources: a row's offset (s * C * 4
// bytes, the same for the whole wave) goes in a scalar register and the
// lane's channel offset in a vector register, so no 64-bit vector address
// arithmetic is spent per row.  Every byte is touched once: loads and stores
// are non-temporal.  A store whose offset is at or beyond the resource's
// size is dropped by the hardware; lanes without a channel use that.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit access, gfx9 family
constexpr int kNonTemporal = 2;
// Row loads: non-temporal by default.  The backward reads k and v twice
// (prefix pass or training forward, then reverse pass); where the two fit in
// the MALL together those passes load on the default policy instead
// (kLoadKeep), so that the second read finds them there.
enum LoadPolicy : int { kLoadStream = kNonTemporal, kLoadKeep = 0 };
constexpr uint32_t kDropOffset = 0x80000000u;

__device__ __forceinline__ Rsrc make_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, int(bytes), kRsrcWord3);
}

// CPL adjacent floats of one row, loaded/stored with a single vector access.
template <int CPL, int POL = kLoadStream>
__device__ __forceinline__ void load_row(Rsrc r, uint32_t voff, uint32_t soff,
                                         float (&x)[CPL]) {
  if constexpr (CPL == 4) {
    typedef int iv4 __attribute__((ext_vector_type(4)));
    const float4 t = __builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POL));
    x[0] = t.x;
    x[1] = t.y;
    x[2] = t.z;
    x[3] = t.w;
  } else if constexpr (CPL == 2) {
    const float2 t = __builtin_bit_cast(
        float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POL));
    x[0] = t.x;
    x[1] = t.y;
  } else {
    x[0] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POL));
  }
}

template <int CPL>
__device__ __forceinline__ void store_row(Rsrc r, uint32_t voff, uint32_t soff,
                                          const float (&x)[CPL]) {
  if constexpr (CPL == 4) {
    typedef int iv4 __attribute__((ext_vector_type(4)));
    const iv4 t = {__float_as_int(x[0]), __float_as_int(x[1]), __float_as_int(x[2]),
                   __float_as_int(x[3])};
    // A store wider than 8 bytes must not see its data registers rewritten
    // in the next cycle.  The compiler inserts that wait state only when the
    // scalar offset is a constant, so the row offset moves into the vector
    // offset here (with a register soffset the first data register was
    // observed to be overwritten before it was stored).
    __builtin_amdgcn_raw_buffer_store_b128(t, r, voff + soff, 0, kNonTemporal);
  } else if constexpr (CPL == 2) {
    typedef int iv2 __attribute__((ext_vector_type(2)));
    const iv2 t = {__float_as_int(x[0]), __float_as_int(x[1])};
    __builtin_amdgcn_raw_buffer_store_b64(t, r, voff, soff, kNonTemporal);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(x[0]), r, voff, soff, kNonTemporal);
  }
}

// History of `n` tokens (n <= L) of one channel from an empty start,
// evaluated after the last one, with a fixed reference instead of a running
// maximum: token s has log2-weight m_s = k2_s - (n-1-s) w2; with
// P = max_s m_s every term is 2^(m_s - P) <= 1 and the largest is exactly 1,
// so nothing overflows and the sum never underflows to 0.
template <int L, int CPL, bool FULL>
__device__ __forceinline__ Hist summarize(const float (&kk)[L][CPL], const float (&vv)[L][CPL],
                                          int c, int n, float w2) {
  if constexpr (FULL) n = L;
  auto expo = [&](int s) {
    const float m = fmaf(-float(n - 1 - s), w2, kk[s][c]);
    return (FULL || s < n) ? m : kEmptyP;
  };
  float P = kEmptyP;
#pragma unroll
  for (int s = 0; s < L; ++s) P = fmaxf(P, expo(s));
  float A = 0.f, Bd = 0.f;
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const float e = exp2_fast(expo(s) - P);  // exactly 0 for padding tokens
    A = fmaf(e, vv[s][c], A);
    Bd += e;
  }
  return n > 0 ? Hist{A, Bd, P, 0.f} : hist_empty();
}

// Forward read of token t fused with the push (as hist_read_push), also
// returning D_t split as 2^{sc} * den (sc: the scale of the larger of the
// history and the token's own term, which contributes exactly 1 to den),
// 1 / den, and the own term's factor pe, so that p_{t,t} = pe / den.  The
// reverse pass carries g_t / den with "key" sc: the sums over 1 / D_t
// without a logarithm per token.
__device__ __forceinline__ float read_push_ld(Hist& h, float k2, float v, float u2, float w2,
                                              float& sc, float& pe, float& rd) {
  const float base = fmaf(-h.n, w2, h.kr - k2);  // p - k2
  const float dr = base - u2;
  const float dp = base - w2;
  const float er = exp2_fast(-fabsf(dr));
  const float ep = exp2_fast(-fabsf(dp));
  const bool kr_keep = dr >= 0.f;
  const float num = kr_keep ? fmaf(er, v, h.A) : fmaf(er, h.A, v);
  const float den = kr_keep ? (h.Bd + er) : fmaf(er, h.Bd, 1.f);
  const float rden = rcp_fast(den);
  sc = kr_keep ? base + k2 : u2 + k2;
  pe = kr_keep ? er : 1.f;
  rd = rden;
  const bool kp_keep = dp >= 0.f;
  h.A = kp_keep ? fmaf(ep, v, h.A) : fmaf(ep, h.A, v);
  h.Bd = kp_keep ? (h.Bd + ep) : fmaf(ep, h.Bd, 1.f);
  h.kr = kp_keep ? h.kr : k2;
  h.n = kp_keep ? (h.n + 1.f) : 0.f;
  return num * rden;
}

// Rescan of a full wave from its starting history hs, in blocks of kBlk
// tokens, calling emit(s, y, sc, pe, rden) for every token s with, per
// channel, y = WKV_s, and D_s = 2^{sc} / rden split as in read_push_ld with
// own-term factor pe (p_{s,s} = pe * rden).
//
// Within a block, multiplying the history before local token t by 2^{t w2}
// makes every term time-independent: token i enters with exponent
// k2_i + (i+1) w2 and the history with its scale p_h.  Measured from the
// block's middle token a (anchor), token i sits at x_i = (k2_i - k2_a) +
// (i-a) w2 and the history at D = p_h - k2_a - (a+1) w2, each formed with one
// rounding at the size of the difference (at most about 4 w2 apart for terms
// that matter together).  The frame is the larger of the anchor and the
// history; every read and push of the block then costs a single exp2 (the
// bonus term is the token's own term times 2^{u2 - w2}), where the exact
// update needs two plus the anchor bookkeeping.  The block leaves the
// history in anchor form: (k2_a, kBlk-1-a decays) if the anchor was the
// frame, else the history's own anchor plus kBlk decays; the denominator
// stays >= 1.  A block whose terms could leave the float range takes the
// exact update: some lane with its history more than 2^{kBlkBelow} under the
// frame (the empty history of a sequence's first block; a key jump of ~100
// log2 units), a token more than 2^{kBlkAbove} over it, or u2 - w2 > 40.
constexpr int kBlk = 8;
constexpr int kBlkAnchor = kBlk / 2 - 1;
constexpr float kBlkBelow = 100.f;
constexpr float kBlkAbove = 80.f;

template <int L, int CPL, class Emit>
__device__ __forceinline__ void rescan_blocked(Hist (&hs)[CPL], const float (&kk)[L][CPL],
                                               const float (&vv)[L][CPL],
                                               const float (&u2)[CPL],
                                               const float (&w2)[CPL], Emit&& emit) {
  static_assert(L % kBlk == 0, "whole blocks");
  float cb[CPL];
  bool lane_ok = true;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    cb[c] = exp2_fast(u2[c] - w2[c]);
    lane_ok = lane_ok && u2[c] - w2[c] <= 40.f;
  }
#pragma unroll
  for (int j = 0; j < L / kBlk; ++j) {
    constexpr int a = kBlkAnchor;
    float x[kBlk][CPL], D[CPL], Dp[CPL];
    bool ok = lane_ok;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float ka = kk[j * kBlk + a][c];
      float mx = 0.f;  // x_a
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        x[i][c] = fmaf(float(i - a), w2[c], kk[j * kBlk + i][c] - ka);
        mx = fmaxf(mx, x[i][c]);
      }
      D[c] = fmaf(-(hs[c].n + float(a + 1)), w2[c], hs[c].kr - ka);  // p_h - k2_a - (a+1) w2
      Dp[c] = fmaxf(D[c], 0.f);
      ok = ok && D[c] >= -kBlkBelow && mx - Dp[c] <= kBlkAbove;
    }
    if (__all(ok)) {
      float A[CPL], B[CPL], f0[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float sh = exp2_fast(fminf(D[c], 0.f));
        A[c] = hs[c].A * sh;
        B[c] = hs[c].Bd * sh;
        f0[c] = kk[j * kBlk + a][c] + Dp[c];  // frame exponent less (a+1) w2
      }
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        float y[CPL], sc[CPL], pe[CPL], rd[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float e = exp2_fast(x[i][c] - Dp[c]);
          const float eb = e * cb[c];
          const float num = fmaf(eb, vv[j * kBlk + i][c], A[c]);
          const float den = B[c] + eb;
          rd[c] = rcp_fast(den);
          y[c] = num * rd[c];
          sc[c] = fmaf(float(a + 1 - i), w2[c], f0[c]);  // D_i = den 2^{sc}
          pe[c] = eb;
          A[c] = fmaf(e, vv[j * kBlk + i][c], A[c]);
          B[c] += e;
        }
        emit(j * kBlk + i, y, sc, pe, rd);
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const bool hist_frame = D[c] >= 0.f;
        hs[c].A = A[c];
        hs[c].Bd = B[c];
        hs[c].kr = hist_frame ? hs[c].kr : kk[j * kBlk + a][c];
        hs[c].n = hist_frame ? hs[c].n + float(kBlk) : float(kBlk - 1 - a);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        float y[CPL], sc[CPL], pe[CPL], rd[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          y[c] = read_push_ld(hs[c], kk[j * kBlk + i][c], vv[j * kBlk + i][c], u2[c], w2[c],
                              sc[c], pe[c], rd[c]);
        emit(j * kBlk + i, y, sc, pe, rd);
      }
    }
  }
}

// Loads of a wave's rows (FULL: all L of them, else the first n; the rest
// are zero) and its second pass, specialised so that a full wave carries no
// per-row checks.  issue_rows only issues the loads (nothing here waits for
// them); scale_keys, the first use of the values, converts k to base 2.
template <int L, int CPL, bool FULL, int POL = kLoadStream>
__device__ __forceinline__ void issue_rows(Rsrc rk, Rsrc rv, uint32_t voff, uint32_t row_bytes,
                                           int n, float (&kk)[L][CPL], float (&vv)[L][CPL]) {
#pragma unroll
  for (int s = 0; s < L; ++s) {
    // Full waves issue their loads in blocks of 8 rows (8 of k, then 8 of v),
    // not in the order the scheduler would pick (which left some early v rows
    // to the very end): at 8x1024x768, 17.07 -> 16.85 us.
    if (FULL && s % 8 == 0 && s > 0) __builtin_amdgcn_sched_barrier(0);
    // Rows go through value temporaries: stores into kk/vv from two branches
    // would otherwise be merged into one store through a pointer select,
    // which keeps the arrays out of registers.
    float tk[CPL], tv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) tk[c] = tv[c] = 0.f;
    if (FULL || s < n) {
      load_row<CPL, POL>(rk, voff, uint32_t(s) * row_bytes, tk);
      load_row<CPL, POL>(rv, voff, uint32_t(s) * row_bytes, tv);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      kk[s][c] = tk[c];
      vv[s][c] = tv[c];
    }
  }
}

template <int L, int CPL>
__device__ __forceinline__ void scale_keys(float (&kk)[L][CPL]) {
#pragma unroll
  for (int s = 0; s < L; ++s)
#pragma unroll
    for (int c = 0; c < CPL; ++c) kk[s][c] *= kLog2e;
}

template <int L, int CPL, bool FULL, int POL = kLoadStream>
__device__ __forceinline__ void load_rows(Rsrc rk, Rsrc rv, uint32_t voff, uint32_t row_bytes,
                                          int n, float (&kk)[L][CPL], float (&vv)[L][CPL]) {
  issue_rows<L, CPL, FULL, POL>(rk, rv, voff, row_bytes, n, kk, vv);
  scale_keys<L, CPL>(kk);
}

// Claims the next tile of channel block g for this workgroup (thread 0
// only).  The call's tag is the workspace epoch + 1, read on the device, so a
// launch replayed from a captured graph still gets a fresh tag.  Tiles are
// handed out 0, 1, 2, ... from the block's counter word {tag, count}.
// Returns the tile, or -1 if the workspace was never zero-filled.
__device__ __forceinline__ int claim_tile(uint32_t* hdr, uint64_t* counters, int g,
                                          int n_tiles, int groups, uint32_t& tag) {
  const uint32_t tg = hdr_load(hdr, kHdrEpoch) + 1u;
  uint64_t* ctr = counters + size_t(g) * (kWkv4CounterStride / sizeof(uint64_t));
  // The claim must not be performed before the epoch read has returned
  // (else this workgroup could see an epoch advanced after its claim): tie
  // the increment to the loaded value.
  uint64_t one = 1;
  asm volatile("" : "+v"(one) : "v"(tg));
  uint64_t old = __hip_atomic_fetch_add(ctr, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (uint32_t(old >> 32) != tg) {
    // The word is left over from a call of another shape: raise it to
    // {tag, 0} (earlier tags are smaller) and claim again.
    __hip_atomic_fetch_max(ctr, uint64_t(tg) << 32, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    old = __hip_atomic_fetch_add(ctr, uint64_t(1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int t = uint32_t(old >> 32) == tg ? int(uint32_t(old)) : -1;
  if (t == n_tiles - 1) {
    // Every tile of this block is claimed: prime the counter for the next
    // call, and the block that completes all claims advances the epoch
    // (every workgroup of this call has read it by then).
    __hip_atomic_store(ctr, uint64_t(tg + 1u) << 32, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (hdr_add(hdr, kHdrClaimed, 1u) == uint32_t(groups - 1)) {
      hdr_store(hdr, kHdrClaimed, 0u);
      hdr_store(hdr, kHdrEpoch, tg);
    }
  }
  tag = tg;
  return t;
}

// Shared-memory copy of per-channel histories, [field][channel].
template <int W>
struct HistLds {
  float f[4][W];
  __device__ __forceinline__ Hist get(int ch) const {
    return Hist{f[0][ch], f[1][ch], f[2][ch], f[3][ch]};
  }
  __device__ __forceinline__ void put(int ch, const Hist& h) {
    f[0][ch] = h.A;
    f[1][ch] = h.Bd;
    f[2][ch] = h.kr;
    f[3][ch] = h.n;
  }
};

}  // namespace scan
}  // namespace rwkv
