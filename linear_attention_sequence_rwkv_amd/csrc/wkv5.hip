// Eagle (RWKV-5) matrix-state WKV forward for gfx950.
//
// What is computed: [Eagle-Finch] "RWKV-5 Eagle and RWKV-6 Finch" (ql.gl
// blog), section "Eagle: extending vector memory to matrix memory":
//   s' = diag(w) s + k^T v,   wkv' = s + diag(u) k^T v,
// read by the receptance like a query.  Per (batch, head) the state s is
// D x D (D = 64), indexed [key i][value j]; diag(w) scales key rows.
//
// Chunked form (chunks of L = 64 tokens; tau, sigma are positions in the
// chunk, S the state at the chunk start).  Unrolling the recurrence,
//   o_tau = r_tau (diag(w^tau) S)
//         + sum_{sigma<tau} (sum_i r_tau[i] w_i^(tau-1-sigma) k_sigma[i]) v_sigma
//         + (sum_i r_tau[i] u_i k_tau[i]) v_tau,
//   S_next = diag(w^L) S + sum_sigma diag(w^(L-1-sigma)) k_sigma^T v_sigma.
// With rt = r (.) w^(tau-32) and kt = k (.) w^(31-sigma) (per element, a
// mid-chunk reference keeps both factors within w^(+-32)), the chunk is four
// dense products on bf16 MFMA with fp32 accumulation:
//   A  = strict_lower(rt kt^T) + diag(beta)         (64 x 64)
//   O  = A V + rt (diag(w^32) S)                    (64 x DV per workgroup)
//   S' = diag(w^32) (diag(w^32) S + kt^T V)         (64 x DV, kept in fp32)
// since w^(63-sigma) = w^32 w^(31-sigma).
// The factorisation needs w^(-32) and w^(31) inside bf16/fp32 range, i.e.
// |log2 w| <= 3.6 for every channel of the head; a head outside that range
// runs the exact fp32 recurrence instead (one branch per workgroup).
#include "eagle_common.h"
#include "wkv_device.h"
#include "wkv_internal.h"

#include <stdlib.h>

#include <algorithm>

namespace rwkv {

namespace {

using namespace eagle;

// Largest |log2 w| for which w^(-32) and w^31 stay far inside fp32/bf16 range.
constexpr float kMaxLog2Decay = 3.6f;

template <int DV>
struct alignas(16) Lds {
  __bf16 rt[kL][kPad];    // rt[tau][i]
  __bf16 kt[kL][kPad];    // kt[sigma][i]
  __bf16 ktt[kD][kPad];   // kt^T[i][sigma]
  __bf16 vt[DV][kPad];    // v^T[j][sigma]
  __bf16 sp[DV][kPad];    // (diag(w^32) S)^T[j][i]
  float l2w[kD];          // log2 w_i
  float w32[kD];          // w_i^32
  float scratch[4][kD];   // the exact recurrence's per-token vectors
  float beta[kL];
  float u[kD];
  int fallback;
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

// Scale one chunk into LDS: rt, kt, kt^T, v^T, beta.  Tokens past T were
// loaded as zeros, so they add nothing to any product.
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
  *reinterpret_cast<bf16x8*>(&s.rt[tau][d0]) = rt0;
  *reinterpret_cast<bf16x8*>(&s.rt[tau][d0 + 8]) = rt1;
  *reinterpret_cast<bf16x8*>(&s.kt[tau][d0]) = kt0;
  *reinterpret_cast<bf16x8*>(&s.kt[tau][d0 + 8]) = kt1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s.ktt[d0 + e][tau] = kt0[e];
    s.ktt[d0 + 8 + e][tau] = kt1[e];
  }
  const uint32_t vw[8] = {x.v0.x, x.v0.y, x.v0.z, x.v0.w, x.v1.x, x.v1.y, x.v1.z, x.v1.w};
  constexpr int VPT = DV / 4;  // value dims per thread
  // v is already bf16: its halves go to v^T as they are
  uint16_t(*vt)[kPad] = reinterpret_cast<uint16_t(*)[kPad]>(&s.vt[0][0]);
#pragma unroll
  for (int e = 0; e < VPT / 2; ++e) {
    vt[VPT * q4 + 2 * e][tau] = uint16_t(vw[e]);
    vt[VPT * q4 + 2 * e + 1][tau] = uint16_t(vw[e] >> 16);
  }
  // the four threads of a token sit in adjacent lanes of one wave
  bpart += __shfl_xor(bpart, 1);
  bpart += __shfl_xor(bpart, 2);
  if (q4 == 0) s.beta[tau] = bpart;
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

  // log2 w, the powers used every chunk, and the range check that picks the
  // path.
  if (tid == 0) s.fallback = 0;
  __syncthreads();
  if (tid < kD) {
    const float wi = w[h * kD + tid];
    s.u[tid] = u[h * kD + tid];
    const float l2w = __log2f(wi);
    s.l2w[tid] = l2w;
    s.w32[tid] = exp2f(32.f * l2w);
    if (!(fabsf(l2w) <= kMaxLog2Decay)) atomicOr(&s.fallback, 1);  // also catches NaN, w<=0
  }
  __syncthreads();
  if (s.fallback) {
    // the exact recurrence runs the whole sequence in the first segment
    if (seg == 0) eagle_recurrent_slice<DV>(T, H, b, h, j0, r, k, v, w, u, o, s_in, s_out, s);
    return;
  }

  const int row = lane & 15;         // MFMA operand row/column of this lane
  const int kq = 8 * (lane >> 4);    // first K element of this lane in a 32-wide step
  const int crow = 4 * (lane >> 4);  // first accumulator row of this lane
  const size_t sbase = size_t(bh) * kD * kD;  // state s[i][j] at sbase + i*kD + j

  // S lives in registers (wave q: key rows 16q..16q+15); S' = diag(w^32) S
  // goes to LDS, transposed, for the inter-chunk product.
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
        pk[rr] = to_bf16(sacc[jb][rr] * s.w32[i]);
      }
      *reinterpret_cast<bf16x4*>(&s.sp[16 * jb + row][16 * q + crow]) = pk;
    }
  };
  write_sp();

  StageConsts f;
  stage_consts(f, s);
  const int n_chunks = (T + kL - 1) / kL;
  const int c_begin = seg * seg_chunks;
  const int c_end = min(n_chunks, c_begin + seg_chunks);
  // o offsets of this lane within a chunk: tokens 16 q + crow + rr
  uint32_t ooff[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
    ooff[rr] = uint32_t(((16 * q + crow + rr) * H * kD + j0 + row) * 4);
  ChunkRegs cur, nxt;
  load_chunk<DV>(cur, c_begin * kL, T, H, b, h, j0, r, k, v);
  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * kL;
    const int n_last = (s_out && c == n_chunks - 1 && T - t0 < kL) ? T - t0 : 0;
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
      const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&s.rt[16 * q + row][32 * ks + kq]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s.kt[16 * nb + row][32 * ks + kq]);
        acc[nb] = mfma(a, bb, acc[nb]);
      }
    }
    // Causal mask and the bonus on the diagonal, in registers.  The pair of
    // sigma tiles (2ks, 2ks+1) held by a lane is directly an A operand of a
    // 32-wide K step, with K ordered as sigma = 32ks + crow + 0..3, then
    // 32ks + 16 + crow + 0..3; V below is read in the same order.
    const int tau_l = 16 * q + row;
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

    // O = A' V + rt S'  (16 tokens x DV value columns per wave).
    floatx4 oacc[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) oacc[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const __bf16* vr = &s.vt[16 * jb + row][32 * ks + crow];
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 16);
        const bf16x8 bb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[jb] = mfma(ap[ks], bb, oacc[jb]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s.rt[16 * q + row][32 * ks + kq]);
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&s.sp[16 * jb + row][32 * ks + kq]);
        oacc[jb] = mfma(a, bb, oacc[jb]);
      }
    }
    {
      const Rsrc ro = chunk_rsrc(o, t0, T, H, b, h, 4);  // rows past T are dropped
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(oacc[jb][rr]), ro, ooff[rr],
                                                64 * jb, kNonTemporal);
    }

    // S <- diag(w^32) (diag(w^32) S + kt^T V) for key rows 16q..16q+15.  A
    // ragged final chunk of n tokens ends with diag(w^(n-32)) instead, which
    // decays S by w^n and token sigma by w^(n-1-sigma).
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float w32 = s.w32[16 * q + crow + rr];
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sacc[jb][rr] *= w32;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s.ktt[16 * q + row][32 * ks + kq]);
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&s.vt[16 * jb + row][32 * ks + kq]);
        sacc[jb] = mfma(a, bb, sacc[jb]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int i = 16 * q + crow + rr;
      const float post = n_last > 0 ? exp2f(float(n_last - 32) * s.l2w[i]) : s.w32[i];
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sacc[jb][rr] *= post;
    }
    __syncthreads();  // every wave is done with rt, kt, kt^T, vt, sp of this chunk

    write_sp();  // S' for the next chunk
    cur = nxt;
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
// start: S <- w^64 S + kh^T V over its chunks, for one value slice.  Written
// to seg_state[bh][seg] as [key i][value j].
template <int DV>
__global__ __launch_bounds__(256) void wkv5_seg_state(int T, int H, int BH, int seg_chunks,
                                                      int nseg, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v,
                                                      const float* __restrict__ w,
                                                      float* __restrict__ seg_state) {
  constexpr int NS = kD / DV;
  constexpr int NJB = DV / 16;
  __shared__ __attribute__((aligned(16))) __bf16 s_kh[kD][kPad];
  __shared__ __attribute__((aligned(16))) __bf16 s_vt[DV][kPad];
  __shared__ float s_l2w[kD];
  __shared__ float s_w64[kD];
  __shared__ int s_fallback;
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
  const int row = lane & 15, kq = 8 * (lane >> 4), crow = 4 * (lane >> 4);
  if (tid == 0) s_fallback = 0;
  __syncthreads();
  if (tid < kD) {
    const float l2w = __log2f(w[h * kD + tid]);
    s_l2w[tid] = l2w;
    s_w64[tid] = exp2f(64.f * l2w);
    if (!(fabsf(l2w) <= kMaxLog2Decay)) atomicOr(&s_fallback, 1);
  }
  __syncthreads();
  if (s_fallback) return;  // that head runs the exact recurrence in one piece
  const int tau = tid >> 2, q4 = tid & 3, d0 = 16 * q4;
  float fh[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) fh[e] = exp2f(float(63 - tau) * s_l2w[d0 + e]);
  floatx4 sacc[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) sacc[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int c_begin = seg * seg_chunks;
  for (int c = c_begin; c < c_begin + seg_chunks; ++c) {
    // every chunk here is whole: only the last segment reaches the end of T
    const size_t off = ((size_t(b) * T + size_t(c) * kL + tau) * H + h) * kD;
    const uint4* kp = reinterpret_cast<const uint4*>(k + off + d0);
    const uint4 k0 = kp[0], k1 = kp[1];
    uint4 v0, v1 = uint4{0u, 0u, 0u, 0u};
    if constexpr (DV == 64) {
      v0 = *reinterpret_cast<const uint4*>(v + off + 16 * q4);
      v1 = *reinterpret_cast<const uint4*>(v + off + 16 * q4 + 8);
    } else if constexpr (DV == 32) {
      v0 = *reinterpret_cast<const uint4*>(v + off + j0 + 8 * q4);
    } else {
      const uint2 t2 = *reinterpret_cast<const uint2*>(v + off + j0 + 4 * q4);
      v0 = uint4{t2.x, t2.y, 0u, 0u};
    }
    const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_kh[d0 + 2 * e][tau] = to_bf16(lo_half(kw[e]) * fh[2 * e]);
      s_kh[d0 + 2 * e + 1][tau] = to_bf16(hi_half(kw[e]) * fh[2 * e + 1]);
    }
    const uint32_t vw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    constexpr int VPT = DV / 4;
#pragma unroll
    for (int e = 0; e < VPT / 2; ++e) {
      s_vt[VPT * q4 + 2 * e][tau] = to_bf16(lo_half(vw[e]));
      s_vt[VPT * q4 + 2 * e + 1][tau] = to_bf16(hi_half(vw[e]));
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float d64 = s_w64[16 * q + crow + rr];
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sacc[jb][rr] *= d64;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s_kh[16 * q + row][32 * ks + kq]);
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&s_vt[16 * jb + row][32 * ks + kq]);
        sacc[jb] = mfma(a, bb, sacc[jb]);
      }
    }
    __syncthreads();
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
// eight (with 32-column slices the best was 166 us).  RWKV_WKV5_SEGS
// overrides (tests, sweeps).
constexpr int64_t kTargetWorkgroups = 512;

int wkv5_segments(int64_t BH, int64_t T, int ns) {
  const int64_t n_chunks = (T + kL - 1) / kL;
  const int64_t per_seg = (BH + 7) / 8 * 8 * ns;
  int64_t nseg = (kTargetWorkgroups + per_seg - 1) / per_seg;
  if (const char* env = getenv("RWKV_WKV5_SEGS")) nseg = atoi(env);
  nseg = std::max<int64_t>(1, std::min<int64_t>(nseg, n_chunks / 4));
  const int64_t seg_chunks = (n_chunks + nseg - 1) / nseg;
  return int((n_chunks + seg_chunks - 1) / seg_chunks);
}

int wkv5_dv() {
  if (const char* env = getenv("RWKV_WKV5_DV")) {
    const int dv = atoi(env);
    return dv == 16 || dv == 64 ? dv : 32;
  }
  return 64;  // whole heads: the intra-chunk products are not repeated per slice
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
