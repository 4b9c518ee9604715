// Finch (RWKV-6) matrix-state WKV forward for gfx950: the Eagle recurrence
// with a decay per token and key channel.
//
// What is computed: [Eagle-Finch] "RWKV-5 Eagle and RWKV-6 Finch" (ql.gl
// blog), section "Finch: making the recurrence respond to the input": the
// Eagle update s' = diag(w) s + k^T v, read out as r (s + diag(u) k^T v),
// with the decay w_t now depending on the token.  Token t's decay multiplies
// the state before its own k^T v is added.
//
// Chunked form (64-token chunks; tau, sigma positions in the chunk; S the
// state at the chunk start; c_tau[i] = sum_{j<tau} log2 w_j[i], so c is
// non-increasing and c_0 = 0):
//   o_tau = r_tau diag(2^c_tau) S
//         + sum_{sigma<tau} (sum_i r_tau[i] k_sigma[i] 2^(c_tau - c_{sigma+1})[i]) v_sigma
//         + (sum_i r_tau[i] u[i] k_tau[i]) v_tau,
//   S_next = diag(2^c_64) S + sum_sigma diag(2^(c_64 - c_{sigma+1})) k_sigma^T v_sigma.
// A decay per token can span any range over a chunk, so one reference point
// (the Eagle kernel's mid-chunk factorisation) could overflow.  The chunk is
// cut into four 16-token blocks, one per wave (wave q owns queries 16q..):
//   * key block b < q: keys scaled by 2^(c_{16b+16} - c_{sigma+1}) and the
//     queries by 2^(c_tau - c_{16b+16}), both factors <= 1;
//   * the diagonal block b = q: a mid-block reference 16q+8, both factors
//     within 2^(8 * 15) as long as every |log2 w| <= 15 in the chunk; a chunk
//     with a faster decay computes its diagonal blocks exactly in fp32;
//   * the inter-chunk term uses r 2^c_tau and the update k 2^(c_64 - c_{sigma+1}),
//     factors <= 1.
// Every product runs on bf16 MFMA with fp32 accumulation; S stays fp32.
#include "eagle_common.h"
#include "wkv_device.h"
#include "wkv_internal.h"

#include <stdlib.h>

#include <algorithm>

namespace rwkv {

namespace {

using namespace eagle;

constexpr int kCPad = 68;                // fp32 row length of the log-decay prefix table (16-byte rows;
                                         // columns 64..67 of rows 0..63 hold the prefix's segment
                                         // totals, of row 64 the per-wave range flags)
constexpr float kMaxDiagLog2 = 15.f;     // fast diagonal blocks need every |log2 w| <= this
constexpr float kMinLog2Decay = -126.f;  // log2 w below this counts as this (2^-126: no memory)

// Per-channel ratios of decay powers for a chunk whose decays all satisfy
// |log2 w| <= 15: every power a product needs is then one power within 8
// tokens of a block middle (finite in fp32) times some of these:
//   2^(c_{16b+16} - c_{s+1}) = 2^(c_{16b+8} - c_{s+1}) g_blk[b],
//   2^(c_64 - c_{s+1})       = 2^(c_{16b+16} - c_{s+1}) h_blk[b],
//   2^(c_t - c_ref)          = (2^(c_t - c_{16q+8}) q_start[q]) q_ref[q][m].
// The query factor for a reference before the block goes through the
// block's first token: q_start and q_ref are both <= 1, so their product
// with 2^(c_t - c_{16q+8}) (up to 2^120) flushes to zero only where the
// true factor is itself below the float range (a direct ratio
// 2^(c_{16q+8} - c_ref) could flush while the factor is as large as 2^-6).
// Ratios that no product uses (a reference after the block) may be inf.
struct DecayTables {
  float g_blk[4][kD];     // 2^(c_{16b+16} - c_{16b+8})
  float h_blk[4][kD];     // 2^(c_64 - c_{16b+16})
  float q_ref[4][4][kD];  // [q][m]: 2^(c_{16q} - c_ref), ref = 16m+16 (m < 3) or 0 (m = 3)
  float q_start[4][kD];   // 2^(c_{16q+8} - c_{16q}), in [2^-120, 1]
  float cmid[4][kD];      // c_{16b+8}
};

template <int DV>
struct alignas(16) LdsF {
  __bf16 rr[kL][kPad];   // r, raw [tau][i]
  __bf16 kb[kL][kPad];   // k 2^(c_{block end} - c_{sigma+1}) [sigma][i]
  __bf16 kd[kL][kPad];   // k 2^(c_{block mid} - c_{sigma+1}), or raw k for exact diagonals
  __bf16 kh[kL][kPad];   // k 2^(c_64 - c_{sigma+1}) [sigma][i]
  __bf16 v[kL][kPad];    // v [sigma][j], DV columns
  __bf16 sp[DV][kPad];   // S^T [j][i]
  float c[kL + 1][kCPad];
  DecayTables tab;        // fast chunks only
  float beta[kL];
  float u[kD];  // 16-byte aligned: the members before it are multiples of 16 bytes
};
// Two workgroups per CU share its 160 KB of LDS (nothing else of the kernel
// is in LDS: at 80 KB + 16 B the compiler drops to one workgroup per CU and
// spends the freed registers).
static_assert(sizeof(LdsF<64>) <= 80 * 1024, "two Finch workgroups per CU");

// This thread's 16 decay factors (token tid/4, channels 16*(tid%4)..).
struct ChunkW {
  float4 a, b, c, d;
};

__device__ __forceinline__ void load_w(ChunkW& x, int t0, int T, int H, int b, int h,
                                       const float* __restrict__ w) {
  const int tid = threadIdx.x;
  const int tau = tid >> 2, q4 = tid & 3;
  if (t0 + tau < T) {
    const float4* p =
        reinterpret_cast<const float4*>(w + ((size_t(b) * T + t0 + tau) * H + h) * kD + 16 * q4);
    x.a = p[0];
    x.b = p[1];
    x.c = p[2];
    x.d = p[3];
  } else {
    // past the end: no decay, so the chunk's end state is the last token's
    const float4 one = {1.f, 1.f, 1.f, 1.f};
    x.a = x.b = x.c = x.d = one;
  }
}

// The segment pass's decays (whole chunks only) through a buffer resource;
// live = false issues the same loads through an empty resource (zeros, no
// memory traffic).
__device__ __forceinline__ void load_w_seg(ChunkW& x, int t0, int T, int H, int b, int h,
                                           const float* __restrict__ w, bool live) {
  const int tid = threadIdx.x;
  const int tau = tid >> 2, q4 = tid & 3;
  const Rsrc rw = chunk_rsrc(w, t0, T, H, b, h, 4, live);
  const uint32_t off = uint32_t((tau * H * kD + 16 * q4) * 4);
  auto f4 = [](uint4 u) {
    return float4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                  __uint_as_float(u.w)};
  };
  x.a = f4(load16(rw, off));
  x.b = f4(load16(rw, off + 16));
  x.c = f4(load16(rw, off + 32));
  x.d = f4(load16(rw, off + 48));
}

// Exclusive prefix c[tau][i] of log2 w over the chunk's tokens.  Returns
// whether some |log2 w| exceeds the fast diagonal's range (block-wide).
typedef float CTable[kL + 1][kCPad];

// With `tab`, a fast chunk's ratio tables are filled from the same sums, by
// the thread that owns (channel, block).
__device__ __forceinline__ bool decay_prefix(const ChunkW& x, CTable& c, DecayTables* tab) {
  const int tid = threadIdx.x;
  const int tau = tid >> 2, d0 = 16 * (tid & 3);
  const float wv[16] = {x.a.x, x.a.y, x.a.z, x.a.w, x.b.x, x.b.y, x.b.z, x.b.w,
                        x.c.x, x.c.y, x.c.z, x.c.w, x.d.x, x.d.y, x.d.z, x.d.w};
  int fast_ok = 1;
  float l2[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    l2[e] = fmaxf(__log2f(wv[e]), kMinLog2Decay);
    fast_ok &= l2[e] >= -kMaxDiagLog2;
  }
#pragma unroll
  for (int e = 0; e < 16; e += 4)
    *reinterpret_cast<float4*>(&c[tau + 1][d0 + e]) =
        float4{l2[e], l2[e + 1], l2[e + 2], l2[e + 3]};
  if (tid < kD) c[0][tid] = 0.f;
  // Whether some decay of the chunk is outside the fast range, over the
  // workgroup: a ballot per wave, kept in the spare cells c[kL][kD + wave]
  // (row kL's padding columns hold nothing else).  __syncthreads_or would
  // take 256 more bytes of LDS, past what two Finch workgroups per CU leave.
  const int wave = tid >> 6;
  const bool wave_any = __ballot(!fast_ok) != 0;
  if ((tid & 63) == 0) c[kL][kD + wave] = wave_any ? 1.f : 0.f;
  __syncthreads();
  const bool exact = c[kL][kD] + c[kL][kD + 1] + c[kL][kD + 2] + c[kL][kD + 3] != 0.f;
  // per channel: four threads each take 16 rows and scan them in registers,
  // then add the totals of the segments before theirs (kept in the rows'
  // padding columns: segment sg of channel ch at c[ch][kD + sg])
  const int ch = tid & 63, sg = tid >> 6;
  float run[16];
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    acc += c[16 * sg + j + 1][ch];
    run[j] = acc;
  }
  c[ch][kD + sg] = acc;
  __syncthreads();
  float tot[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) tot[j] = c[ch][kD + j];
  float off = 0.f;
  for (int j = 0; j < sg; ++j) off += tot[j];
#pragma unroll
  for (int j = 0; j < 16; ++j) c[16 * sg + j + 1][ch] = run[j] + off;
  if (tab && !exact) {
    // the same sums as the table entries c_{16b+8}, c_{16b+16}, c_64
    float cend[4];  // c_{16m+16}
    float om = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      cend[m] = om + tot[m];
      om += tot[m];
    }
    const float cm = run[7] + off;  // c_{16 sg + 8}; off = c_{16 sg}
    tab->cmid[sg][ch] = cm;
    tab->g_blk[sg][ch] = exp2_fast(run[15] + off - cm);
    tab->h_blk[sg][ch] = exp2_fast(cend[3] - (run[15] + off));
    tab->q_start[sg][ch] = exp2_fast(cm - off);
#pragma unroll
    for (int m = 0; m < 4; ++m) tab->q_ref[sg][m][ch] = exp2_fast(off - (m < 3 ? cend[m] : 0.f));
  }
  __syncthreads();
  return exact;
}

// Scaled copies of one chunk into LDS (the decay prefix must be in place),
// all row-major: products over sigma read kh and v with the transpose load.
template <int DV>
__device__ __forceinline__ void stage_chunk_f(const ChunkRegs& x, bool exact, LdsF<DV>& s) {
  const int tid = threadIdx.x;
  const int tau = tid >> 2, q4 = tid & 3;
  const int d0 = 16 * q4;
  const int blk = tau >> 4;
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
  *reinterpret_cast<uint4*>(&s.rr[tau][d0]) = x.r0;
  *reinterpret_cast<uint4*>(&s.rr[tau][d0 + 8]) = x.r1;
  float bpart = 0.f;
  bf16x8 kba, kbb, kda, kdb, kha, khb;
  // this token's prefix and, on fast chunks, the block's reference and
  // ratios for the 16 channels (and u): 16-byte reads
  float ct[16], cm[16], gb[16], hb[16], uu[16];
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const float4 a = *reinterpret_cast<const float4*>(&s.u[d0 + e]);
    uu[e] = a.x, uu[e + 1] = a.y, uu[e + 2] = a.z, uu[e + 3] = a.w;
  }
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const float4 a = *reinterpret_cast<const float4*>(&s.c[tau + 1][d0 + e]);
    ct[e] = a.x;
    ct[e + 1] = a.y;
    ct[e + 2] = a.z;
    ct[e + 3] = a.w;
  }
  if (!exact) {
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const float4 a = *reinterpret_cast<const float4*>(&s.tab.cmid[blk][d0 + e]);
      const float4 g4 = *reinterpret_cast<const float4*>(&s.tab.g_blk[blk][d0 + e]);
      const float4 h4 = *reinterpret_cast<const float4*>(&s.tab.h_blk[blk][d0 + e]);
      cm[e] = a.x;
      cm[e + 1] = a.y;
      cm[e + 2] = a.z;
      cm[e + 3] = a.w;
      gb[e] = g4.x;
      gb[e + 1] = g4.y;
      gb[e + 2] = g4.z;
      gb[e + 3] = g4.w;
      hb[e] = h4.x;
      hb[e + 1] = h4.y;
      hb[e + 2] = h4.z;
      hb[e + 3] = h4.w;
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int i = d0 + e;
    const float ct1 = ct[e];
    float fkb, fkd, fkh;
    if (exact) {
      fkb = exp2_fast(s.c[16 * blk + 16][i] - ct1);
      fkd = exp2_fast(s.c[16 * blk + 8][i] - ct1);
      fkh = exp2_fast(s.c[kL][i] - ct1);
    } else {
      fkd = exp2_fast(cm[e] - ct1);
      fkb = fkd * gb[e];
      fkh = fkb * hb[e];
    }
    const __bf16 vkb = to_bf16(kv[e] * fkb);
    const __bf16 vkd = exact ? to_bf16(kv[e]) : to_bf16(kv[e] * fkd);
    const __bf16 vkh = to_bf16(kv[e] * fkh);
    if (e < 8) {
      kba[e] = vkb;
      kda[e] = vkd;
      kha[e] = vkh;
    } else {
      kbb[e - 8] = vkb;
      kdb[e - 8] = vkd;
      khb[e - 8] = vkh;
    }
    bpart = fmaf(rv[e] * uu[e], kv[e], bpart);
  }
  *reinterpret_cast<bf16x8*>(&s.kb[tau][d0]) = kba;
  *reinterpret_cast<bf16x8*>(&s.kb[tau][d0 + 8]) = kbb;
  *reinterpret_cast<bf16x8*>(&s.kd[tau][d0]) = kda;
  *reinterpret_cast<bf16x8*>(&s.kd[tau][d0 + 8]) = kdb;
  *reinterpret_cast<bf16x8*>(&s.kh[tau][d0]) = kha;
  *reinterpret_cast<bf16x8*>(&s.kh[tau][d0 + 8]) = khb;
  // v is already bf16: DV / 4 value dims of this token go in as loaded
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

// Queries of this lane's B operand (token tau, channels i0..i0+7) scaled by
// 2^(c_tau - c_ref).
template <int DV>
__device__ __forceinline__ bf16x8 scaled_queries(const LdsF<DV>& s, int tau, int i0, int ref) {
  const bf16x8 raw = *reinterpret_cast<const bf16x8*>(&s.rr[tau][i0]);
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    out[e] = to_bf16(float(raw[e]) * exp2_fast(s.c[tau][i0 + e] - s.c[ref][i0 + e]));
  return out;
}

// Workgroup: 4 waves; (batch, head, slice of DV value columns), placed as in
// the Eagle kernel.
template <int DV>
__global__ __launch_bounds__(256, 2) void wkv6_fwd_chunked(
    int T, int H, int BH, const uint16_t* __restrict__ r, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ w,
    const float* __restrict__ u, float* __restrict__ o, const float* s_in, float* s_out,
    int seg_chunks, int pieces, const float* __restrict__ seg_state) {
  constexpr int NS = kD / DV;
  constexpr int NJB = DV / 16;
  __shared__ LdsF<DV> s;
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
  // Wave w of the workgroup takes query block (w + blockIdx) mod 4 (the same
  // for every workgroup of an XCD): the last block has four key blocks of
  // score work and the first one, and which wave takes the heavy block
  // matters (same results; 4x4096x32x64: 147.5 us with block w, 145.7 us with
  // this, 145.9 us with block 3 - w, 150.1 us with a rotation that differs
  // between the workgroups of one XCD).
  const int q = __builtin_amdgcn_readfirstlane(((tid >> 6) + (int(blockIdx.x) & 3)) & 3);
  const int row = lane & 15;
  const int kq = 8 * (lane >> 4);
  const int crow = 4 * (lane >> 4);
  const size_t sbase = size_t(bh) * kD * kD;

  if (tid < kD) s.u[tid] = u[h * kD + tid];

  floatx4 sacc[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      sacc[jb][rr] = s_in ? s_in[sbase + size_t(16 * q + crow + rr) * kD + j0 + 16 * jb + row]
                          : 0.f;
  // A later segment starts from the local end states of the earlier
  // segments' pieces (`pieces` per segment), in order:
  // S <- diag(2^L_piece) S + S_piece, L_piece the piece's summed log2 decay.
  if (seg > 0) {
    const int npieces = (int(gridDim.x) / per_seg - 1) * pieces;
    for (int sg = 0; sg < seg * pieces; ++sg) {
      const float* src = seg_state + (size_t(bh) * npieces + sg) * (kD * kD + kD);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 16 * q + crow + rr;
        const float d = exp2_fast(src[kD * kD + i]);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
          sacc[jb][rr] = fmaf(d, sacc[jb][rr], src[size_t(i) * kD + j0 + 16 * jb + row]);
      }
    }
  }
  auto write_sp = [&]() {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      bf16x4 pk;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) pk[rr] = to_bf16(sacc[jb][rr]);
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
  // A chunk's o goes out at the top of the next chunk, after the loads of
  // that chunk (one chunk ahead) and before their wait, which then leaves the
  // stores in flight (loads and stores share one completion counter; stores
  // at the end of a chunk were covered by that wait).  The first pass's
  // deferred store goes through an empty resource.
  auto store_o = [&](const floatx4 (&x)[NJB], int t0, bool live) {
    const Rsrc ro = chunk_rsrc(o, t0, T, H, b, h, 4, live);  // rows past T are dropped
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(x[jb][rr]), ro, ooff[rr], 64 * jb,
                                              kStoreAux);
  };
  floatx4 opend[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) opend[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
  ChunkRegs cur, nxt;
  ChunkW wc, wn;
  load_chunk<DV>(cur, c_begin * kL, T, H, b, h, j0, r, k, v);
  load_w(wc, c_begin * kL, T, H, b, h, w);
  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * kL;
    store_o(opend, c > c_begin ? t0 - kL : t0, c > c_begin);
    // The decay prefix and staging (latency-bound, barrier-separated) run at
    // raised issue priority over the other workgroup's products on the same
    // SIMDs (4x4096x32x64: 164.9 -> 162.7 us).
    __builtin_amdgcn_s_setprio(2);
    const bool exact = decay_prefix(wc, s.c, &s.tab);
    stage_chunk_f(cur, exact, s);
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    if (c + 1 < c_end) {
      load_chunk<DV>(nxt, t0 + kL, T, H, b, h, j0, r, k, v);
      load_w(wn, t0 + kL, T, H, b, h, w);
    }

    // A^T: key blocks nb <= q against this wave's 16 queries (column
    // tau = 16q + row of the lane, rows sigma = 16nb + crow .. +3).  The
    // lane's scaled queries r 2^c_tau for the inter-chunk product share its
    // operand position and are formed here too.
    const int tau_l = 16 * q + row;
    // acc[nb]: key blocks before the wave's own; dacc: the diagonal block
    // (kept apart so that no register array is indexed by the wave number)
    floatx4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    floatx4 dacc = {0.f, 0.f, 0.f, 0.f};
    bf16x8 ainter[2];
    if (!exact) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int i0 = 32 * ks + kq;
        const bf16x8 raw = *reinterpret_cast<const bf16x8*>(&s.rr[tau_l][i0]);
        auto ld8 = [](const float* p, float (&x)[8]) {
          const float4 a = *reinterpret_cast<const float4*>(p);
          const float4 b = *reinterpret_cast<const float4*>(p + 4);
          x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w;
          x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
        };
        // qb: r 2^(c_tau - c_{16q+8}) (diagonal block); qs: r 2^(c_tau - c_{16q})
        float ctl[8], cml[8], qst[8], qb[8], qs[8];
        ld8(&s.c[tau_l][i0], ctl);
        ld8(&s.tab.cmid[q][i0], cml);
        ld8(&s.tab.q_start[q][i0], qst);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qb[e] = float(raw[e]) * exp2_fast(ctl[e] - cml[e]);
          qs[e] = qb[e] * qst[e];
        }
#pragma unroll
        for (int nb = 0; nb < 3; ++nb)
          if (nb < q) {
            float qr[8];
            ld8(&s.tab.q_ref[q][nb][i0], qr);
            bf16x8 bq;
#pragma unroll
            for (int e = 0; e < 8; ++e) bq[e] = to_bf16(qs[e] * qr[e]);
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s.kb[16 * nb + row][i0]);
            acc[nb] = mfma(a, bq, acc[nb]);
          }
        float q0[8];
        ld8(&s.tab.q_ref[q][3][i0], q0);
        bf16x8 bq;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bq[e] = to_bf16(qb[e]);
          ainter[ks][e] = to_bf16(qs[e] * q0[e]);
        }
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s.kd[16 * q + row][i0]);
        dacc = mfma(a, bq, dacc);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int i0 = 32 * ks + kq;
#pragma unroll
        for (int nb = 0; nb < 3; ++nb)
          if (nb < q) {
            const bf16x8 bq = scaled_queries(s, tau_l, i0, 16 * nb + 16);
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&s.kb[16 * nb + row][i0]);
            acc[nb] = mfma(a, bq, acc[nb]);
          }
        // r 2^c_tau (row 0 of the prefix table is zero)
        ainter[ks] = scaled_queries(s, tau_l, i0, 0);
      }
      // diagonal block in fp32: sum_i r[tau][i] k[sigma][i] 2^(c_tau - c_{sigma+1})[i]
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int sig = 16 * q + crow + rr;
        float a = 0.f;
        if (sig < tau_l) {
          for (int i = 0; i < kD; ++i)
            a = fmaf(float(s.rr[tau_l][i]) * float(s.kd[sig][i]),
                     exp2_fast(s.c[tau_l][i] - s.c[sig + 1][i]), a);
        }
        dacc[rr] = a;
      }
    }

    // Causal mask and the bonus, in registers (as in the Eagle kernel).
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

    // O = A' V + (r 2^c) S, and S <- diag(2^c_64) S + kh^T V for key rows
    // 16q..16q+15; the products over sigma share their V operands.
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float dall = exp2_fast(s.c[kL][16 * q + crow + rr]);
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sacc[jb][rr] *= dall;
    }
    floatx4 oacc[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) oacc[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 kop = sigma_operand(s.kh, 32 * ks, 16 * q, lane);
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const bf16x8 vop = sigma_operand(s.v, 32 * ks, 16 * jb, lane);
        oacc[jb] = mfma(ap[ks], vop, oacc[jb]);
        sacc[jb] = mfma(kop, vop, sacc[jb]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&s.sp[16 * jb + row][32 * ks + kq]);
        oacc[jb] = mfma(ainter[ks], bb, oacc[jb]);
      }
    }
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) opend[jb] = oacc[jb];
    __syncthreads();  // every wave is done with this chunk's LDS

    write_sp();
    cur = nxt;
    wc = wn;
  }
  if (c_end > c_begin) store_o(opend, (c_end - 1) * kL, true);
  if (s_out && c_end == n_chunks) {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        s_out[sbase + size_t(16 * q + crow + rr) * kD + j0 + 16 * jb + row] = sacc[jb][rr];
  }
}

// Local end state of one time segment (all but the last) from a zero start,
// and the segment's summed log2 decay per key channel, for one value slice:
// seg_state[bh][seg] holds S[i][j] (64 x 64) then L[i] (64).  The next
// chunk's k, v and decays load while this one is processed.
template <int DV>
__global__ __launch_bounds__(256) void wkv6_seg_state(int T, int H, int BH, int seg_chunks,
                                                      int npieces, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v,
                                                      const float* __restrict__ w,
                                                      float* __restrict__ seg_state) {
  constexpr int NS = kD / DV;
  constexpr int NJB = DV / 16;
  __shared__ __attribute__((aligned(16))) CTable s_c;
  __shared__ __attribute__((aligned(16))) __bf16 s_kh[kL][kPad];
  __shared__ __attribute__((aligned(16))) __bf16 s_v[kL][kPad];
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
  const int tau = tid >> 2, q4 = tid & 3, d0 = 16 * q4;
  floatx4 sacc[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) sacc[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
  float ltot = 0.f;  // thread tid < 64: channel tid
  const int c_begin = seg * seg_chunks;
  const int c_end = c_begin + seg_chunks;  // every chunk here is whole
  // One chunk: S <- diag(2^c_64) S + kh^T V, and the chunk's summed decay.
  auto chunk_step = [&](const ChunkRegs& x, const ChunkW& xw) {
    decay_prefix(xw, s_c, nullptr);
    const uint32_t kw[8] = {x.k0.x, x.k0.y, x.k0.z, x.k0.w, x.k1.x, x.k1.y, x.k1.z, x.k1.w};
    float ce[16], ct[16];  // c_64 and this token's c_{tau+1}, 16-byte reads
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const float4 a = *reinterpret_cast<const float4*>(&s_c[kL][d0 + e]);
      const float4 t = *reinterpret_cast<const float4*>(&s_c[tau + 1][d0 + e]);
      ce[e] = a.x, ce[e + 1] = a.y, ce[e + 2] = a.z, ce[e + 3] = a.w;
      ct[e] = t.x, ct[e + 1] = t.y, ct[e + 2] = t.z, ct[e + 3] = t.w;
    }
    bf16x8 kh0, kh1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float kvv = (e & 1) ? hi_half(kw[e >> 1]) : lo_half(kw[e >> 1]);
      const __bf16 y = to_bf16(kvv * exp2_fast(ce[e] - ct[e]));
      if (e < 8)
        kh0[e] = y;
      else
        kh1[e - 8] = y;
    }
    *reinterpret_cast<bf16x8*>(&s_kh[tau][d0]) = kh0;
    *reinterpret_cast<bf16x8*>(&s_kh[tau][d0 + 8]) = kh1;
    if constexpr (DV == 64) {
      *reinterpret_cast<uint4*>(&s_v[tau][16 * q4]) = x.v0;
      *reinterpret_cast<uint4*>(&s_v[tau][16 * q4 + 8]) = x.v1;
    } else if constexpr (DV == 32) {
      *reinterpret_cast<uint4*>(&s_v[tau][8 * q4]) = x.v0;
    } else {
      *reinterpret_cast<uint2*>(&s_v[tau][4 * q4]) = uint2{x.v0.x, x.v0.y};
    }
    if (tid < kD) ltot += s_c[kL][tid];
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float dall = exp2_fast(s_c[kL][16 * q + crow + rr]);
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sacc[jb][rr] *= dall;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 kop = sigma_operand(s_kh, 32 * ks, 16 * q, lane);
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
        sacc[jb] = mfma(kop, sigma_operand(s_v, 32 * ks, 16 * jb, lane), sacc[jb]);
    }
    __syncthreads();
  };
  // Two register buffers in turn: each chunk's loads go out before the
  // previous chunk's decay prefix, so they have a whole chunk's work to land
  // (with one buffer and a copy between, the copy waits for them; loads
  // issued after the staging barrier had only the products to hide behind).
  // A load past the piece goes through an empty resource, so every pass
  // issues the same loads and each wait stays with its own chunk.
  // 4x4096x32x64: 149.6 -> 147.5 us per call.  (The same in the Eagle
  // segment pass, whose chunks carry less work, measured 0.2-1.1 us slower.)
  ChunkRegs ca, cb;
  ChunkW wa, wb;
  load_chunk<DV, false>(ca, c_begin * kL, T, H, b, h, j0, nullptr, k, v);
  load_w_seg(wa, c_begin * kL, T, H, b, h, w, true);
  for (int c = c_begin; c < c_end; c += 2) {
    const bool more = c + 1 < c_end;
    const int t1 = (more ? c + 1 : c) * kL;
    load_chunk<DV, false>(cb, t1, T, H, b, h, j0, nullptr, k, v, more);
    load_w_seg(wb, t1, T, H, b, h, w, more);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before this chunk is staged
    chunk_step(ca, wa);
    if (!more) break;
    const bool more2 = c + 2 < c_end;
    const int t2 = (more2 ? c + 2 : c) * kL;
    load_chunk<DV, false>(ca, t2, T, H, b, h, j0, nullptr, k, v, more2);
    load_w_seg(wa, t2, T, H, b, h, w, more2);
    __builtin_amdgcn_sched_barrier(0);
    chunk_step(cb, wb);
  }
  float* dst = seg_state + (size_t(bh) * npieces + seg) * (kD * kD + kD);
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      dst[size_t(16 * q + crow + rr) * kD + j0 + 16 * jb + row] = sacc[jb][rr];
  if (slice == 0 && tid < kD) dst[kD * kD + tid] = ltot;
}

// Time segments per head (as for Eagle): about two workgroups per CU over the
// launch, segments of at least four chunks; kTuneWkv6Segs overrides.
constexpr int64_t kTargetWorkgroups = 512;

// Pieces per segment for the segment pass: halves of segments of 8 or more
// chunks, each with its local end state and summed decay, folded in order
// (4x4096x32x64: 151.4 -> 149.6 us; four pieces 152.2).  The Eagle segment
// pass, with less work per chunk, measured slower split.
int wkv6_pieces(int64_t seg_chunks) { return seg_chunks % 2 == 0 && seg_chunks >= 8 ? 2 : 1; }

int wkv6_dv() { return tuning(kTuneWkv6Dv) == 32 ? 32 : 64; }

int wkv6_segments(int64_t BH, int64_t T, int ns) {
  const int64_t n_chunks = (T + kL - 1) / kL;
  const int64_t per_seg = (BH + 7) / 8 * 8 * ns;
  int64_t nseg = (kTargetWorkgroups + per_seg - 1) / per_seg;
  if (const int o = tuning(kTuneWkv6Segs)) nseg = o;
  nseg = std::max<int64_t>(1, std::min<int64_t>(nseg, n_chunks / 4));
  const int64_t seg_chunks = (n_chunks + nseg - 1) / nseg;
  return int((n_chunks + seg_chunks - 1) / seg_chunks);
}

template <int DV>
hipError_t launch_wkv6(int64_t T, int64_t H, int64_t BH, const uint16_t* r, const uint16_t* k,
                       const uint16_t* v, const float* w, const float* u, float* o,
                       const float* s_in, float* s_out, float* seg_state, hipStream_t stream) {
  constexpr int NS = kD / DV;
  const int nseg = wkv6_segments(BH, T, NS);
  const int64_t n_chunks = (T + kL - 1) / kL;
  const int seg_chunks = int((n_chunks + nseg - 1) / nseg);
  const int pieces = wkv6_pieces(seg_chunks);
  const int npieces = (nseg - 1) * pieces;
  const unsigned per_seg = unsigned((BH + 7) / 8 * 8 * NS);
  if (nseg > 1) {
    hipLaunchKernelGGL(wkv6_seg_state<DV>, dim3(per_seg * unsigned(npieces)), dim3(256), 0,
                       stream, int(T), int(H), int(BH), seg_chunks / pieces, npieces, k, v, w,
                       seg_state);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(wkv6_fwd_chunked<DV>, dim3(per_seg * unsigned(nseg)), dim3(256), 0, stream,
                     int(T), int(H), int(BH), r, k, v, w, u, o, s_in, s_out, seg_chunks, pieces,
                     seg_state);
  return hipGetLastError();
}

}  // namespace

size_t wkv6_workspace_bytes(int64_t B, int64_t T, int64_t H) {
  const int nseg = wkv6_segments(B * H, T, kD / wkv6_dv());
  const int64_t n_chunks = (T + kL - 1) / kL;
  const int pieces = wkv6_pieces((n_chunks + nseg - 1) / nseg);
  return size_t(B * H) * size_t(nseg - 1) * size_t(pieces) * (kD * kD + kD) * sizeof(float);
}

hipError_t wkv6_forward_launch(int64_t B, int64_t T, int64_t H, const uint16_t* r,
                               const uint16_t* k, const uint16_t* v, const float* w,
                               const float* u, float* o, const float* s_in, float* s_out,
                               void* ws, hipStream_t stream) {
  float* seg_state = static_cast<float*>(ws);
  if (wkv6_dv() == 32)
    return launch_wkv6<32>(T, H, B * H, r, k, v, w, u, o, s_in, s_out, seg_state, stream);
  return launch_wkv6<64>(T, H, B * H, r, k, v, w, u, o, s_in, s_out, seg_state, stream);
}

}  // namespace rwkv
