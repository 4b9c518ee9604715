// Eagle (RWKV-5) matrix-state WKV forward for gfx950.
//
// What is computed: [Eagle-Finch] "RWKV-5 Eagle and RWKV-6 Finch" (ql.gl
// blog), section "Eagle: extending vector memory to matrix memory":
//   s' = diag(w) s + k^T v,   wkv' = s + diag(u) k^T v,
// read by the receptance like a query.  Per (batch, head) the state s is
// D x D (D = 64), indexed [key i][value j]; diag(w) scales key rows.  The
// section parameterises the decay as w = exp(-exp(omega)), in (0, 1).
//
// Chunked form (chunks of L = 64 tokens; tau, sigma are positions in the
// chunk, S the state at the chunk start).  Unrolling the recurrence,
//   o_tau = r_tau (diag(w^tau) S)
//         + sum_{sigma<tau} (sum_i r_tau[i] w_i^(tau-1-sigma) k_sigma[i]) v_sigma
//         + (sum_i r_tau[i] u_i k_tau[i]) v_tau,
//   S_next = diag(w^L) S + sum_sigma diag(w^(L-1-sigma)) k_sigma^T v_sigma.
// Every product runs on bf16 MFMA with fp32 accumulation; S stays fp32.
// How the decay powers are split between queries and keys depends on the
// head's fastest decay (one branch per workgroup):
//
// * Mid-chunk reference, when every |log2 w| <= 3.6.  With
//   rt = r (.) w^(tau-32) and kt = k (.) w^(31-sigma), both within w^(+-32),
//   the chunk is four dense products:
//     A  = strict_lower(rt kt^T) + diag(beta)         (64 x 64)
//     O  = A V + rt (diag(w^32) S)                    (64 x DV per workgroup)
//     S' = diag(w^32) (diag(w^32) S + kt^T V)
//   since w^(63-sigma) = w^32 w^(31-sigma).
// * 16-token blocks, for faster decays.  Wave q owns the queries
//   tau = 16q + p.  A key block nb < q is referred to its end 16nb + 16: keys
//   k w^(15 - sigma%16), queries r w^p w^(16(q-1-nb)), both factors <= 1.
//   The diagonal block is referred to its middle, k w^(7 - sigma%16) and
//   r w^(p-8), within w^(+-8): that needs every |log2 w| <= 15, and a head
//   with a faster decay sums its diagonal blocks exactly in fp32 instead.
//   The inter-chunk term uses r w^tau (<= 1) against S itself, the update
//   k w^(63-sigma) (<= 1).  As w is the same for every token, each of these
//   factors is fixed per thread.
// * A head with some w outside [0, 1] (or NaN), outside that
//   parameterisation, runs the exact fp32 recurrence: one workgroup per
//   head and value slice over the whole sequence.
// On the chunked paths a decay below 2^-126 acts as 2^-126.
#include "eagle_common.h"
#include "wkv_device.h"
#include "wkv_internal.h"

#include <stdlib.h>

#include <algorithm>

namespace rwkv {

namespace {

using namespace eagle;

constexpr float kMaxLog2Decay = 3.6f;    // mid-chunk reference: every |log2 w| <= this
constexpr float kMaxDiagLog2 = 15.f;     // fast diagonal blocks: every |log2 w| <= this
constexpr float kMinLog2Decay = -126.f;  // log2 w below this counts as this

// A head's path, from its decays (bits, ORed over its channels).
constexpr int kModeBlocks = 1;     // some |log2 w| > kMaxLog2Decay: 16-token blocks
constexpr int kModeExactDiag = 2;  // some |log2 w| > kMaxDiagLog2: exact diagonal blocks
constexpr int kModeRecurrent = 4;  // some w outside [0, 1], or NaN

// log2 w of channel threadIdx.x (< kD) of head h; its mode bits are ORed
// into *mode.
__device__ __forceinline__ float head_decay(const float* __restrict__ w, int h, int* mode) {
  const float wi = w[h * kD + threadIdx.x];
  const float l2w = fmaxf(__log2f(wi), kMinLog2Decay);  // log2(0) = -inf
  int m = 0;
  if (!(wi >= 0.f && wi <= 1.f)) m |= kModeRecurrent;
  if (!(fabsf(l2w) <= kMaxLog2Decay)) m |= kModeBlocks;
  if (!(fabsf(l2w) <= kMaxDiagLog2)) m |= kModeExactDiag;
  if (m) atomicOr(mode, m);
  return l2w;
}

template <int DV>
struct alignas(16) Lds {
  // the chunk's scaled operands, [token][channel]: mid-chunk path a[0] = rt,
  // a[1] = kt; block path a[0] = r, a[1] = kb (keys to their block's end),
  // a[2] = kd (to its middle; raw k for exact diagonals), a[3] = kh (to the
  // chunk's end)
  __bf16 a[4][kL][kPad];
  __bf16 v[kL][kPad];     // v[sigma][j], DV columns
  __bf16 sp[DV][kPad];    // S^T[j][i] as the inter-chunk product reads it
  float l2w[kD];          // log2 w_i
  float w32[kD];          // w_i^32
  float w16m[4][kD];      // w_i^(16m)
  float wpow[15][kD];     // w_i^d (exact diagonal blocks)
  float scratch[4][kD];   // the exact recurrence's per-token vectors
  float beta[kL];
  float u[kD];
  int mode;
};

// Exact fp32 recurrence for one (batch, head, value slice): lane j < DV
// keeps the state column s[:, j] in registers.
template <int DV>
__device__ void eagle_recurrent_slice(int T, int H, int b, int h, int j0,
                                     const uint16_t* __restrict__ r,
                                     const uint16_t* __restrict__ k,
                                     const uint16_t* __restrict__ v,
                                     const float* __restrict__ w,
                                     const float* __restrict__ u, float* __restrict__ o,
                                     const float* s_in, float* s_out,
                                     Lds<DV>& s) {
  float* s_r = s.scratch[0];
  float* s_k = s.scratch[1];
  float* s_w = s.scratch[2];
  float* s_u = s.scratch[3];
  const int tid = threadIdx.x;
  if (tid < kD) {
    s_w[tid] = w[h * kD + tid];
    s_u[tid] = u[h * kD + tid];
  }
  const size_t sbase = (size_t(b) * H + h) * kD * kD + j0 + tid;  // s[i][j0+tid] at + i*kD
  float S[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) S[i] = (s_in && tid < DV) ? s_in[sbase + size_t(i) * kD] : 0.f;
  for (int t = 0; t < T; ++t) {
    const size_t off = ((size_t(b) * T + t) * H + h) * kD;
    __syncthreads();
    if (tid < kD) {
      s_r[tid] = bf16_to_f32(r[off + tid]);
      s_k[tid] = bf16_to_f32(k[off + tid]);
    }
    __syncthreads();
    if (tid < DV) {
      const float vj = bf16_to_f32(v[off + j0 + tid]);
      float acc = 0.f, beta = 0.f;
#pragma unroll
      for (int i = 0; i < kD; ++i) {
        const float ri = s_r[i], ki = s_k[i];
        acc = fmaf(ri, S[i], acc);
        beta = fmaf(ri * s_u[i], ki, beta);
        S[i] = fmaf(s_w[i], S[i], ki * vj);
      }
      o[off + j0 + tid] = fmaf(beta, vj, acc);
    }
  }
  if (s_out && tid < DV) {
#pragma unroll
    for (int i = 0; i < kD; ++i) s_out[sbase + size_t(i) * kD] = S[i];
  }
}

// Decay factors and bonus of the 16 channels this thread scales.  The
// thread's token position in a chunk never changes, so they are computed once
// and kept in registers (reading them from the shared table would put every
// lane of a 16-token column on one LDS bank).
struct StageConsts {
  float fr[16];  // w^(tau-32)
  float fk[16];  // w^(31-tau)
};

template <int DV>
__device__ __forceinline__ void stage_consts(StageConsts& c, const Lds<DV>& s) {
  const int tid = threadIdx.x;
  const int tau = tid >> 2, d0 = 16 * (tid & 3);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float l2 = s.l2w[d0 + e];
    c.fr[e] = exp2f(float(tau - 32) * l2);
    c.fk[e] = exp2f(float(31 - tau) * l2);
  }
}

// Mid-chunk path: scale one chunk into LDS: rt, kt, v (all row-major: products over sigma
// read them with the transpose load) and beta.  Tokens past T were loaded as
// zeros, so they add nothing to any product.
template <int DV>
__device__ __forceinline__ void stage_chunk(const ChunkRegs& x, const StageConsts& f,
                                            Lds<DV>& s) {
  const int tid = threadIdx.x;
  const int tau = tid >> 2, q4 = tid & 3;
  const int d0 = 16 * q4;
  float rv[16], kv[16];
  const uint32_t rw[8] = {x.r0.x, x.r0.y, x.r0.z, x.r0.w, x.r1.x, x.r1.y, x.r1.z, x.r1.w};
  const uint32_t kw[8] = {x.k0.x, x.k0.y, x.k0.z, x.k0.w, x.k1.x, x.k1.y, x.k1.z, x.k1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    rv[2 * e] = lo_half(rw[e]);
    rv[2 * e + 1] = hi_half(rw[e]);
    kv[2 * e] = lo_half(kw[e]);
    kv[2 * e + 1] = hi_half(kw[e]);
  }
  float bpart = 0.f;
  bf16x8 rt0, rt1, kt0, kt1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    rt0[e] = to_bf16(rv[e] * f.fr[e]);
    rt1[e] = to_bf16(rv[8 + e] * f.fr[8 + e]);
    kt0[e] = to_bf16(kv[e] * f.fk[e]);
    kt1[e] = to_bf16(kv[8 + e] * f.fk[8 + e]);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) bpart = fmaf(rv[e] * s.u[d0 + e], kv[e], bpart);
  *reinterpret_cast<bf16x8*>(&s.a[0][tau][d0]) = rt0;
  *reinterpret_cast<bf16x8*>(&s.a[0][tau][d0 + 8]) = rt1;
  *reinterpret_cast<bf16x8*>(&s.a[1][tau][d0]) = kt0;
  *reinterpret_cast<bf16x8*>(&s.a[1][tau][d0 + 8]) = kt1;
  // v is already bf16: DV / 4 value dims of this token go in as loaded
  if constexpr (DV == 64) {
    *reinterpret_cast<uint4*>(&s.v[tau][16 * q4]) = x.v0;
    *reinterpret_cast<uint4*>(&s.v[tau][16 * q4 + 8]) = x.v1;
  } else if constexpr (DV == 32) {
    *reinterpret_cast<uint4*>(&s.v[tau][8 * q4]) = x.v0;
  } else {
    *reinterpret_cast<uint2*>(&s.v[tau][4 * q4]) = uint2{x.v0.x, x.v0.y};
  }
  // the four threads of a token sit in adjacent lanes of one wave
  bpart += __shfl_xor(bpart, 1);
  bpart += __shfl_xor(bpart, 2);
  if (q4 == 0) s.beta[tau] = bpart;
}

// Block path: the key factors of the 16 channels this thread stages
// (token tau = tid/4, channels 16 (tid%4) ..), the same for every chunk.
struct BlockStageConsts {
  float fb[16];  // w^(15 - tau%16): to the key's block end
  float fd[16];  // w^(7 - tau%16): to its block middle
  float fh[16];  // w^(63 - tau): to the chunk end
};

template <int DV>
__device__ __forceinline__ void block_stage_consts(BlockStageConsts& c, const Lds<DV>& s) {
  const int tid = threadIdx.x;
  const int tau = tid >> 2, p = tau & 15, d0 = 16 * (tid & 3);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float l2 = s.l2w[d0 + e];
    c.fb[e] = exp2f(float(15 - p) * l2);
    c.fd[e] = exp2f(float(7 - p) * l2);
    c.fh[e] = exp2f(float(63 - tau) * l2);
  }
}

// Block path: one chunk into LDS: raw r, kb, kd (raw k for exact
// diagonals), kh, v and beta.  n_last > 0 marks the sequence's ragged last
// chunk of n_last tokens whose end state is wanted: its update keys carry
// w^(n_last-1-sigma) instead, and 0 past the last token.
template <int DV>
__device__ __forceinline__ void block_stage_chunk(const ChunkRegs& x, const BlockStageConsts& f,
                                                  bool exact_diag, int n_last, Lds<DV>& s) {
  const int tid = threadIdx.x;
  const int tau = tid >> 2, q4 = tid & 3;
  const int d0 = 16 * q4;
  float rv[16], kv[16];
  const uint32_t rw[8] = {x.r0.x, x.r0.y, x.r0.z, x.r0.w, x.r1.x, x.r1.y, x.r1.z, x.r1.w};
  const uint32_t kw[8] = {x.k0.x, x.k0.y, x.k0.z, x.k0.w, x.k1.x, x.k1.y, x.k1.z, x.k1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    rv[2 * e] = lo_half(rw[e]);
    rv[2 * e + 1] = hi_half(rw[e]);
    kv[2 * e] = lo_half(kw[e]);
    kv[2 * e + 1] = hi_half(kw[e]);
  }
  *reinterpret_cast<uint4*>(&s.a[0][tau][d0]) = x.r0;
  *reinterpret_cast<uint4*>(&s.a[0][tau][d0 + 8]) = x.r1;
  bf16x8 kb0, kb1, kd0, kd1, kh0, kh1;
  float bpart = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float fh = f.fh[e];
    if (n_last > 0) fh = tau < n_last ? exp2f(float(n_last - 1 - tau) * s.l2w[d0 + e]) : 0.f;
    const __bf16 xb = to_bf16(kv[e] * f.fb[e]);
    const __bf16 xd = exact_diag ? to_bf16(kv[e]) : to_bf16(kv[e] * f.fd[e]);
    const __bf16 xh = to_bf16(kv[e] * fh);
    if (e < 8) {
      kb0[e] = xb;
      kd0[e] = xd;
      kh0[e] = xh;
    } else {
      kb1[e - 8] = xb;
      kd1[e - 8] = xd;
      kh1[e - 8] = xh;
    }
    bpart = fmaf(rv[e] * s.u[d0 + e], kv[e], bpart);
  }
  *reinterpret_cast<bf16x8*>(&s.a[1][tau][d0]) = kb0;
  *reinterpret_cast<bf16x8*>(&s.a[1][tau][d0 + 8]) = kb1;
  *reinterpret_cast<bf16x8*>(&s.a[2][tau][d0]) = kd0;
  *reinterpret_cast<bf16x8*>(&s.a[2][tau][d0 + 8]) = kd1;
  *reinterpret_cast<bf16x8*>(&s.a[3][tau][d0]) = kh0;
  *reinterpret_cast<bf16x8*>(&s.a[3][tau][d0 + 8]) = kh1;
  if constexpr (DV == 64) {
    *reinterpret_cast<uint4*>(&s.v[tau][16 * q4]) = x.v0;
    *reinterpret_cast<uint4*>(&s.v[tau][16 * q4 + 8]) = x.v1;
  } else if constexpr (DV == 32) {
    *reinterpret_cast<uint4*>(&s.v[tau][8 * q4]) = x.v0;
  } else {
    *reinterpret_cast<uint2*>(&s.v[tau][4 * q4]) = uint2{x.v0.x, x.v0.y};
  }
  bpart += __shfl_xor(bpart, 1);
  bpart += __shfl_xor(bpart, 2);
  if (q4 == 0) s.beta[tau] = bpart;
}

__device__ __forceinline__ void ld8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w;
  x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
}

// Workgroup: 4 waves; (batch, head, slice of DV value columns).  blockIdx
// places the 64/DV slices of a head 8 apart, so that they land on the same
// XCD (dispatch is round-robin over 8 XCDs) and share r, k reads in its L2.
template <int DV>
__global__ __launch_bounds__(256, 2) void wkv5_fwd_chunked(
    int T, int H, int BH, const uint16_t* __restrict__ r, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ w,
    const float* __restrict__ u, float* __restrict__ o, const float* s_in, float* s_out,
    int seg_chunks, const float* __restrict__ seg_state) {
  constexpr int NS = kD / DV;  // slices per head
  constexpr int NJB = DV / 16; // 16-wide value tiles per slice
  __shared__ Lds<DV> s;
  const int per_seg = (BH + 7) / 8 * 8 * NS;  // workgroups per time segment
  const int seg = blockIdx.x / per_seg;
  const int bx = blockIdx.x - seg * per_seg;
  const int bh = (bx / (8 * NS)) * 8 + (bx & 7);
  const int slice = (bx >> 3) % NS;
  if (bh >= BH) return;
  const int b = bh / H, h = bh - (bh / H) * H;
  const int j0 = slice * DV;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = __builtin_amdgcn_readfirstlane(tid >> 6);

  // log2 w, the powers used every chunk, and the head's path.
  if (tid == 0) s.mode = 0;
  __syncthreads();
  if (tid < kD) {
    s.u[tid] = u[h * kD + tid];
    const float l2w = head_decay(w, h, &s.mode);
    s.l2w[tid] = l2w;
    s.w32[tid] = exp2f(32.f * l2w);
  }
  __syncthreads();
  const int mode = __builtin_amdgcn_readfirstlane(s.mode);
  if (mode & kModeRecurrent) {
    // the exact recurrence runs the whole sequence in the first segment
    if (seg == 0) eagle_recurrent_slice<DV>(T, H, b, h, j0, r, k, v, w, u, o, s_in, s_out, s);
    return;
  }
  const bool blocks = (mode & kModeBlocks) != 0;
  if (blocks) {
    // the block path's per-channel power tables (filling them on every head
    // cost the mid-chunk path 3 us of the 4x4096x32x64 call)
    if (tid < kD) {
      const float l2w = s.l2w[tid];
#pragma unroll
      for (int m = 0; m < 4; ++m) s.w16m[m][tid] = exp2f(float(16 * m) * l2w);
#pragma unroll
      for (int d = 0; d < 15; ++d) s.wpow[d][tid] = exp2f(float(d) * l2w);
    }
    __syncthreads();  // uniform: the whole workgroup is on one path
  }

  const int row = lane & 15;         // MFMA operand row/column of this lane
  const int kq = 8 * (lane >> 4);    // first K element of this lane in a 32-wide step
  const int crow = 4 * (lane >> 4);  // first accumulator row of this lane
  const size_t sbase = size_t(bh) * kD * kD;  // state s[i][j] at sbase + i*kD + j

  // S lives in registers (wave q: key rows 16q..16q+15) and goes to LDS,
  // transposed, for the inter-chunk product: as diag(w^32) S on the
  // mid-chunk path, as S on the block path.
  floatx4 sacc[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      sacc[jb][rr] = s_in ? s_in[sbase + size_t(16 * q + crow + rr) * kD + j0 + 16 * jb + row]
                          : 0.f;
  // A later segment starts from the earlier segments' local end states,
  // each decayed over the segments after it: S <- w^len S + S_seg.
  if (seg > 0) {
    float dseg[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      dseg[rr] = exp2f(float(seg_chunks * kL) * s.l2w[16 * q + crow + rr]);
    const int nseg = int(gridDim.x) / per_seg;
    for (int sg = 0; sg < seg; ++sg) {
      const float* src = seg_state + (size_t(bh) * (nseg - 1) + sg) * kD * kD;
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          sacc[jb][rr] = fmaf(dseg[rr], sacc[jb][rr],
                              src[size_t(16 * q + crow + rr) * kD + j0 + 16 * jb + row]);
    }
  }
  auto write_sp = [&]() {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 pk;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 16 * q + crow + rr;
        pk[rr] = to_bf16(blocks ? sacc[jb][rr] : sacc[jb][rr] * s.w32[i]);
      }
      *reinterpret_cast<bf16x4*>(&s.sp[16 * jb + row][16 * q + crow]) = pk;
    }
  };
  write_sp();

  const int n_chunks = (T + kL - 1) / kL;
  const int c_begin = seg * seg_chunks;
  const int c_end = min(n_chunks, c_begin + seg_chunks);
  // o offsets of this lane within a chunk: tokens 16 q + crow + rr
  uint32_t ooff[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
    ooff[rr] = uint32_t(((16 * q + crow + rr) * H * kD + j0 + row) * 4);
  const int tau_l = 16 * q + row;  // this lane's query in the score and inter-chunk operands
  auto store_o = [&](const floatx4 (&oacc)[NJB], int t0, bool live = true) {
    const Rsrc ro = chunk_rsrc(o, t0, T, H, b, h, 4, live);  // rows past T are dropped
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(oacc[jb][rr]), ro, ooff[rr],
                                              64 * jb, kStoreAux);
  };
  // The same stores row by row (a row's four 64-byte pieces back to back):
  // the mid-chunk path measured 90.7 -> 89.9 us with it; the block path and
  // the Finch kernel measured slower and keep the column-block order.
  auto store_o_rows = [&](const floatx4 (&oacc)[NJB], int t0, bool live = true) {
    const Rsrc ro = chunk_rsrc(o, t0, T, H, b, h, 4, live);  // rows past T are dropped
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(oacc[jb][rr]), ro, ooff[rr],
                                              64 * jb, kStoreAux);
  };
  // Each path's fixed factors come before the first chunk's loads (issued
  // first, they cost the mid-chunk path 2.3 us of the 4x4096x32x64 call).
  //
  // A chunk's o goes out at the top of the next chunk, right before the
  // wait for that chunk's loads (issued mid-chunk, one chunk ahead), instead
  // of at the end of its own.  Loads and stores share one completion counter:
  // stores at the end of a chunk are still in flight at the next chunk's
  // first use of its inputs, and the wait there also covered them (measured:
  // 95.8 -> 90.6 us at 4x4096x32x64).  Stores issued after the loads are
  // left in flight by that wait.  The first chunk's deferred store goes
  // through an empty resource, so that every pass through the loop issues the
  // same operations and the wait is the same on its first pass.
  ChunkRegs cur, nxt;
  if (blocks) {
    const bool exact_diag = (mode & kModeExactDiag) != 0;
    BlockStageConsts f;
    block_stage_consts(f, s);
    // this lane's query factors: w^p and w^(p-8), p = row, for its channels
    // 32 ks + kq + e
    float fq[16], fdq[16];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float l2 = s.l2w[32 * ks + kq + e];
        fq[8 * ks + e] = exp2f(float(row) * l2);
        fdq[8 * ks + e] = exp2f(float(row - 8) * l2);
      }
    load_chunk<DV>(cur, c_begin * kL, T, H, b, h, j0, r, k, v);
    floatx4 opend[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) opend[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int c = c_begin; c < c_end; ++c) {
      const int t0 = c * kL;
      const int n_last = (s_out && c == n_chunks - 1 && T - t0 < kL) ? T - t0 : 0;
      store_o(opend, c > c_begin ? t0 - kL : t0, c > c_begin);
      block_stage_chunk(cur, f, exact_diag, n_last, s);
      __syncthreads();
      if (c + 1 < c_end) load_chunk<DV>(nxt, t0 + kL, T, H, b, h, j0, r, k, v);

      // A^T: key blocks nb < q (each against the queries referred to its
      // end) and the diagonal block; the inter-chunk queries r w^tau are
      // formed alongside.  Lane: column tau_l, rows sigma = 16nb + crow ..
      floatx4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      floatx4 dacc = {0.f, 0.f, 0.f, 0.f};
      bf16x8 ainter[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int i0 = 32 * ks + kq;
        const bf16x8 raw = *reinterpret_cast<const bf16x8*>(&s.a[0][tau_l][i0]);
        float rq[8];  // r w^p
#pragma unroll
        for (int e = 0; e < 8; ++e) rq[e] = float(raw[e]) * fq[8 * ks + e];
#pragma unroll
        for (int nb = 0; nb < 3; ++nb)
          if (nb < q) {
            float wm[8];
            ld8(&s.w16m[q - 1 - nb][i0], wm);
            bf16x8 bq;
#pragma unroll
            for (int e = 0; e < 8; ++e) bq[e] = to_bf16(rq[e] * wm[e]);
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s.a[1][16 * nb + row][i0]);
            acc[nb] = mfma(a, bq, acc[nb]);
          }
        float wq[8];
        ld8(&s.w16m[q][i0], wq);
#pragma unroll
        for (int e = 0; e < 8; ++e) ainter[ks][e] = to_bf16(rq[e] * wq[e]);
        if (!exact_diag) {
          bf16x8 bd;
#pragma unroll
          for (int e = 0; e < 8; ++e) bd[e] = to_bf16(float(raw[e]) * fdq[8 * ks + e]);
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s.a[2][16 * q + row][i0]);
          dacc = mfma(a, bd, dacc);
        }
      }
      if (exact_diag) {
        // sum_i r[tau][i] k[sigma][i] w_i^(tau-1-sigma), raw r and k in fp32
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int sig = 16 * q + crow + rr;
          float a = 0.f;
          if (sig < tau_l) {
            const int d = tau_l - 1 - sig;  // 0 .. 14
            for (int i = 0; i < kD; ++i)
              a = fmaf(float(s.a[0][tau_l][i]) * float(s.a[2][sig][i]), s.wpow[d][i], a);
          }
          dacc[rr] = a;
        }
      }

      // Causal mask and the bonus on the diagonal, in registers.
      const float beta = s.beta[tau_l];
      bf16x8 ap[2];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int sig = 16 * nb + crow + rr;
          const float sc = nb == q ? dacc[rr] : (nb < 3 ? acc[nb < 3 ? nb : 0][rr] : 0.f);
          const float val = sig < tau_l ? sc : (sig == tau_l ? beta : 0.f);
          ap[nb >> 1][(nb & 1) * 4 + rr] = to_bf16(val);
        }

      // O = A' V + (r w^tau) S and S <- diag(w^64) S + kh^T V (w^n_last for a
      // ragged last chunk whose end state is wanted); the two products over
      // sigma share their V operands.
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float l2 = s.l2w[16 * q + crow + rr];
        const float dall = exp2f(float(n_last > 0 ? n_last : kL) * l2);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) sacc[jb][rr] *= dall;
      }
      floatx4 oacc[NJB];
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) oacc[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 kop = sigma_operand(s.a[3], 32 * ks, 16 * q, lane);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          const bf16x8 vop = sigma_operand(s.v, 32 * ks, 16 * jb, lane);
          oacc[jb] = mfma(ap[ks], vop, oacc[jb]);
          sacc[jb] = mfma(kop, vop, sacc[jb]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&s.sp[16 * jb + row][32 * ks + kq]);
          oacc[jb] = mfma(ainter[ks], bb, oacc[jb]);
        }
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) opend[jb] = oacc[jb];
      __syncthreads();  // every wave is done with this chunk's LDS

      write_sp();  // S for the next chunk
      cur = nxt;
    }
    if (c_end > c_begin) store_o(opend, (c_end - 1) * kL);
  } else {
    StageConsts f;
    stage_consts(f, s);
    load_chunk<DV>(cur, c_begin * kL, T, H, b, h, j0, r, k, v);
    floatx4 opend[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) opend[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int c = c_begin; c < c_end; ++c) {
      const int t0 = c * kL;
      const int n_last = (s_out && c == n_chunks - 1 && T - t0 < kL) ? T - t0 : 0;
      store_o_rows(opend, c > c_begin ? t0 - kL : t0, c > c_begin);
      stage_chunk(cur, f, s);
      __syncthreads();
      if (c + 1 < c_end) load_chunk<DV>(nxt, t0 + kL, T, H, b, h, j0, r, k, v);

      // A^T = kt rt^T for all four sigma blocks against this wave's 16 tokens
      // (blocks after the wave's own are masked to zero below; computing them
      // costs a few MFMAs but no branches): lane holds column tau = 16q + row,
      // rows sigma = 16nb + crow .. +3.
      floatx4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f},
                        {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&s.a[0][tau_l][32 * ks + kq]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s.a[1][16 * nb + row][32 * ks + kq]);
          acc[nb] = mfma(a, bb, acc[nb]);
        }
      }
      // Causal mask and the bonus on the diagonal, in registers.  The pair of
      // sigma tiles (2ks, 2ks+1) held by a lane is directly an A operand of a
      // 32-wide K step, with K ordered as sigma = 32ks + crow + 0..3, then
      // 32ks + 16 + crow + 0..3: the order of sigma_operand.
      const float beta = s.beta[tau_l];
      bf16x8 ap[2];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int sig = 16 * nb + crow + rr;
          const float val = sig < tau_l ? acc[nb][rr] : (sig == tau_l ? beta : 0.f);
          ap[nb >> 1][(nb & 1) * 4 + rr] = to_bf16(val);
        }

      // O = A' V + rt S' (16 tokens x DV value columns per wave) and
      // S <- diag(w^32) (diag(w^32) S + kt^T V) for key rows 16q..16q+15: the
      // two products over sigma share their V operands.  A ragged final chunk
      // of n tokens ends with diag(w^(n-32)) instead, which decays S by w^n and
      // token sigma by w^(n-1-sigma).
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float w32 = s.w32[16 * q + crow + rr];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) sacc[jb][rr] *= w32;
      }
      floatx4 oacc[NJB];
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) oacc[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 kop = sigma_operand(s.a[1], 32 * ks, 16 * q, lane);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          const bf16x8 vop = sigma_operand(s.v, 32 * ks, 16 * jb, lane);
          oacc[jb] = mfma(ap[ks], vop, oacc[jb]);
          sacc[jb] = mfma(kop, vop, sacc[jb]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s.a[0][tau_l][32 * ks + kq]);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&s.sp[16 * jb + row][32 * ks + kq]);
          oacc[jb] = mfma(a, bb, oacc[jb]);
        }
      }
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) opend[jb] = oacc[jb];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 16 * q + crow + rr;
        const float post = n_last > 0 ? exp2f(float(n_last - 32) * s.l2w[i]) : s.w32[i];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) sacc[jb][rr] *= post;
      }
      __syncthreads();  // every wave is done with rt, kt, v, sp of this chunk

      write_sp();  // S' for the next chunk
      cur = nxt;
    }
    if (c_end > c_begin) store_o_rows(opend, (c_end - 1) * kL);
  }
  if (s_out && c_end == n_chunks) {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        s_out[sbase + size_t(16 * q + crow + rr) * kD + j0 + 16 * jb + row] = sacc[jb][rr];
  }
}

// Local end state of one time segment (all but the last), from a zero
// start, over its chunks, for one value slice: S <- diag(w^64) S + kh^T V
// with kh = k w^(63-sigma) (every factor <= 1, for any decay in [0, 1]);
// the next chunk's k, v load while this one multiplies.  Written to
// seg_state[bh][seg] as [key i][value j].  Heads on the exact recurrence
// need none.
template <int DV>
__global__ __launch_bounds__(256) void wkv5_seg_state(int T, int H, int BH, int seg_chunks,
                                                      int nseg, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v,
                                                      const float* __restrict__ w,
                                                      float* __restrict__ seg_state) {
  constexpr int NS = kD / DV;
  constexpr int NJB = DV / 16;
  __shared__ __attribute__((aligned(16))) __bf16 s_kh[kL][kPad];
  __shared__ __attribute__((aligned(16))) __bf16 s_v[kL][kPad];
  __shared__ float s_l2w[kD];
  __shared__ int s_mode;
  const int per_seg = (BH + 7) / 8 * 8 * NS;
  const int seg = blockIdx.x / per_seg;
  const int bx = blockIdx.x - seg * per_seg;
  const int bh = (bx / (8 * NS)) * 8 + (bx & 7);
  const int slice = (bx >> 3) % NS;
  if (bh >= BH) return;
  const int b = bh / H, h = bh - (bh / H) * H;
  const int j0 = slice * DV;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 15, crow = 4 * (lane >> 4);
  if (tid == 0) s_mode = 0;
  __syncthreads();
  if (tid < kD) s_l2w[tid] = head_decay(w, h, &s_mode);
  __syncthreads();
  if (s_mode & kModeRecurrent) return;  // that head runs the exact recurrence in one piece
  const int tau = tid >> 2, q4 = tid & 3, d0 = 16 * q4;
  float fh[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) fh[e] = exp2f(float(63 - tau) * s_l2w[d0 + e]);
  float w64[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) w64[rr] = exp2f(64.f * s_l2w[16 * q + crow + rr]);
  floatx4 sacc[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) sacc[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int c_begin = seg * seg_chunks;
  const int c_end = c_begin + seg_chunks;  // every chunk here is whole
  ChunkRegs cur, nxt;
  load_chunk<DV, false>(cur, c_begin * kL, T, H, b, h, j0, nullptr, k, v);
  for (int c = c_begin; c < c_end; ++c) {
    const uint32_t kw[8] = {cur.k0.x, cur.k0.y, cur.k0.z, cur.k0.w,
                            cur.k1.x, cur.k1.y, cur.k1.z, cur.k1.w};
    bf16x8 kh0, kh1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kh0[2 * e] = to_bf16(lo_half(kw[e]) * fh[2 * e]);
      kh0[2 * e + 1] = to_bf16(hi_half(kw[e]) * fh[2 * e + 1]);
      kh1[2 * e] = to_bf16(lo_half(kw[4 + e]) * fh[8 + 2 * e]);
      kh1[2 * e + 1] = to_bf16(hi_half(kw[4 + e]) * fh[8 + 2 * e + 1]);
    }
    *reinterpret_cast<bf16x8*>(&s_kh[tau][d0]) = kh0;
    *reinterpret_cast<bf16x8*>(&s_kh[tau][d0 + 8]) = kh1;
    if constexpr (DV == 64) {
      *reinterpret_cast<uint4*>(&s_v[tau][16 * q4]) = cur.v0;
      *reinterpret_cast<uint4*>(&s_v[tau][16 * q4 + 8]) = cur.v1;
    } else if constexpr (DV == 32) {
      *reinterpret_cast<uint4*>(&s_v[tau][8 * q4]) = cur.v0;
    } else {
      *reinterpret_cast<uint2*>(&s_v[tau][4 * q4]) = uint2{cur.v0.x, cur.v0.y};
    }
    __syncthreads();
    if (c + 1 < c_end) load_chunk<DV, false>(nxt, (c + 1) * kL, T, H, b, h, j0, nullptr, k, v);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sacc[jb][rr] *= w64[rr];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 kop = sigma_operand(s_kh, 32 * ks, 16 * q, lane);
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
        sacc[jb] = mfma(kop, sigma_operand(s_v, 32 * ks, 16 * jb, lane), sacc[jb]);
    }
    __syncthreads();
    cur = nxt;
  }
  float* dst = seg_state + (size_t(bh) * (nseg - 1) + seg) * kD * kD;
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      dst[size_t(16 * q + crow + rr) * kD + j0 + 16 * jb + row] = sacc[jb][rr];
}

// One token of the recurrence for every (batch, head): lane j keeps the
// state column s[:, j] (read, updated and written back in place).  With
// PER_TOKEN_W (Finch) the decay is this token's [B, H, D] instead of [H, D].
template <bool PER_TOKEN_W>
__global__ __launch_bounds__(64) void wkv5_step_kernel(
    int H, float* __restrict__ S, const uint16_t* __restrict__ r,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ w, const float* __restrict__ u, float* __restrict__ o) {
  __shared__ float s_r[kD], s_k[kD], s_w[kD], s_ru[kD];
  const int bh = blockIdx.x;
  const int h = bh % H;
  const int j = threadIdx.x;
  const size_t off = size_t(bh) * kD;
  float* Sc = S + size_t(bh) * kD * kD + j;
  float col[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) col[i] = Sc[size_t(i) * kD];
  const float rj = bf16_to_f32(r[off + j]);
  const float kj = bf16_to_f32(k[off + j]);
  s_r[j] = rj;
  s_k[j] = kj;
  s_w[j] = PER_TOKEN_W ? w[off + j] : w[h * kD + j];
  s_ru[j] = rj * u[h * kD + j];
  __syncthreads();
  const float vj = bf16_to_f32(v[off + j]);
  float acc = 0.f, beta = 0.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    acc = fmaf(s_r[i], col[i], acc);
    beta = fmaf(s_ru[i], s_k[i], beta);
    col[i] = fmaf(s_w[i], col[i], s_k[i] * vj);
  }
  o[off + j] = fmaf(beta, vj, acc);
#pragma unroll
  for (int i = 0; i < kD; ++i) Sc[size_t(i) * kD] = col[i];
}

}  // namespace

namespace {

// Time segments per head: about two workgroups per CU over the launch,
// segments of at least four chunks.  Measured at B=4 T=4096 H=32 with whole
// heads per workgroup: 242 us in one segment, 128 us in four, 133 us in
// eight (with 32-column slices the best was 166 us).  The kTuneWkv5Segs
// override replaces the target (tests, sweeps).
constexpr int64_t kTargetWorkgroups = 512;

int wkv5_segments(int64_t BH, int64_t T, int ns) {
  const int64_t n_chunks = (T + kL - 1) / kL;
  const int64_t per_seg = (BH + 7) / 8 * 8 * ns;
  int64_t nseg = (kTargetWorkgroups + per_seg - 1) / per_seg;
  if (const int o = tuning(kTuneWkv5Segs)) nseg = o;
  nseg = std::max<int64_t>(1, std::min<int64_t>(nseg, n_chunks / 4));
  const int64_t seg_chunks = (n_chunks + nseg - 1) / nseg;
  return int((n_chunks + seg_chunks - 1) / seg_chunks);
}

int wkv5_dv() {
  // whole heads by default: the intra-chunk products are not repeated per slice
  const int o = tuning(kTuneWkv5Dv);
  return o ? o : 64;
}

}  // namespace

size_t wkv5_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t D) {
  (void)D;
  const int nseg = wkv5_segments(B * H, T, kD / wkv5_dv());
  return size_t(B * H) * size_t(nseg - 1) * kD * kD * sizeof(float);
}

hipError_t wkv5_forward_launch(int64_t B, int64_t T, int64_t H, int64_t D,
                               const uint16_t* r, const uint16_t* k, const uint16_t* v,
                               const float* w, const float* u, float* o, void* ws,
                               const float* s_in, float* s_out, hipStream_t stream) {
  (void)D;
  const int64_t BH = B * H;
  const int dv = wkv5_dv();
  const int ns = kD / dv;
  const int nseg = wkv5_segments(BH, T, ns);
  const int64_t n_chunks = (T + kL - 1) / kL;
  const int seg_chunks = int((n_chunks + nseg - 1) / nseg);
  const unsigned per_seg = unsigned((BH + 7) / 8 * 8 * ns);
  float* seg_state = static_cast<float*>(ws);
  if (nseg > 1) {
    if (dv == 16)
      hipLaunchKernelGGL(wkv5_seg_state<16>, dim3(per_seg * unsigned(nseg - 1)), dim3(256), 0,
                         stream, int(T), int(H), int(BH), seg_chunks, nseg, k, v, w, seg_state);
    else if (dv == 64)
      hipLaunchKernelGGL(wkv5_seg_state<64>, dim3(per_seg * unsigned(nseg - 1)), dim3(256), 0,
                         stream, int(T), int(H), int(BH), seg_chunks, nseg, k, v, w, seg_state);
    else
      hipLaunchKernelGGL(wkv5_seg_state<32>, dim3(per_seg * unsigned(nseg - 1)), dim3(256), 0,
                         stream, int(T), int(H), int(BH), seg_chunks, nseg, k, v, w, seg_state);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(per_seg * unsigned(nseg));
  if (dv == 16)
    hipLaunchKernelGGL(wkv5_fwd_chunked<16>, grid, dim3(256), 0, stream, int(T), int(H), int(BH),
                       r, k, v, w, u, o, s_in, s_out, seg_chunks, seg_state);
  else if (dv == 64)
    hipLaunchKernelGGL(wkv5_fwd_chunked<64>, grid, dim3(256), 0, stream, int(T), int(H), int(BH),
                       r, k, v, w, u, o, s_in, s_out, seg_chunks, seg_state);
  else
    hipLaunchKernelGGL(wkv5_fwd_chunked<32>, grid, dim3(256), 0, stream, int(T), int(H), int(BH),
                       r, k, v, w, u, o, s_in, s_out, seg_chunks, seg_state);
  return hipGetLastError();
}

hipError_t wkv5_step_launch(int64_t B, int64_t H, float* s, const uint16_t* r,
                            const uint16_t* k, const uint16_t* v, const float* w,
                            const float* u, float* o, hipStream_t stream) {
  hipLaunchKernelGGL(wkv5_step_kernel<false>, dim3(unsigned(B * H)), dim3(64), 0, stream, int(H),
                     s, r, k, v, w, u, o);
  return hipGetLastError();
}

hipError_t wkv6_step_launch(int64_t B, int64_t H, float* s, const uint16_t* r,
                            const uint16_t* k, const uint16_t* v, const float* w,
                            const float* u, float* o, hipStream_t stream) {
  hipLaunchKernelGGL(wkv5_step_kernel<true>, dim3(unsigned(B * H)), dim3(64), 0, stream, int(H),
                     s, r, k, v, w, u, o);
  return hipGetLastError();
}

}  // namespace rwkv
