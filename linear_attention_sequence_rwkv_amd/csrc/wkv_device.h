// Device helpers shared by the WKV kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rwkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// "No history yet" scale exponent.  Finite, so that differences of two empty
// scales are 0 rather than NaN; exp2 of anything this negative is exactly 0.
constexpr float kEmptyP = -1.0e38f;

// v_exp_f32: 2^x, about 1 ulp; results below the normal range flush to 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// v_rcp_f32: 1/x, about 1 ulp.
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// ---------------------------------------------------------------------------
// RWKV-4 history arithmetic in the base-2 domain.
//
// A lane's history is (A, Bd): the numerator and denominator sums are A * 2^p
// and Bd * 2^p, with k, w, u pre-multiplied by log2(e).  The scale is carried as an
// anchor: p = kr - n * w2, where kr is a (pre-scaled) key and n an integer
// count of decay steps since it.  Every comparison of two scales is formed
// as fma(-(n_a - n_b), w2, kr_a - kr_b), which rounds once at the size of the
// difference and never accumulates rounding along the sequence: a plain
// running p -= w2 would drift by ulp(|p|) per token.
//
// Each update keeps the larger of the two scales at factor 1, so a single
// exp2 of a non-positive number is needed.  Exact integers up to 2^24 are
// held in the float n.
// ---------------------------------------------------------------------------
struct Hist {
  float A, Bd, kr, n;
};

__device__ __forceinline__ Hist hist_empty() { return Hist{0.f, 0.f, kEmptyP, 0.f}; }

// Scale of the history as a plain exponent (for the recurrent-state ABI).
__device__ __forceinline__ float hist_p(const Hist& h, float w2) { return fmaf(-h.n, w2, h.kr); }

// Output for the current token, (history + 2^(u2+k2) v) / (history + 2^(u2+k2)),
// fused with advancing the history by that token (decay by 2^-w2, then add
// 2^k2 * (v, 1)).  Both exponents share kr - k2.
__device__ __forceinline__ float hist_read_push(Hist& h, float k2, float v, float u2, float w2) {
  const float base = fmaf(-h.n, w2, h.kr - k2);  // p - k2
  const float dr = base - u2;                     // p - (u2 + k2)
  const float dp = base - w2;                     // (p - w2) - k2
  const float er = exp2_fast(-fabsf(dr));
  const float ep = exp2_fast(-fabsf(dp));
  const bool kr_keep = dr >= 0.f;
  const float num = kr_keep ? fmaf(er, v, h.A) : fmaf(er, h.A, v);
  const float den = kr_keep ? (h.Bd + er) : fmaf(er, h.Bd, 1.f);
  const float y = num * rcp_fast(den);
  const bool kp_keep = dp >= 0.f;
  h.A = kp_keep ? fmaf(ep, v, h.A) : fmaf(ep, h.A, v);
  h.Bd = kp_keep ? (h.Bd + ep) : fmaf(ep, h.Bd, 1.f);
  h.kr = kp_keep ? h.kr : k2;
  h.n = kp_keep ? (h.n + 1.f) : 0.f;
  return y;
}

// Concatenate histories: `x` covers an earlier stretch, `y` the `ny` tokens
// right after it (y was accumulated from an empty history).  Decay-then-add
// is associative, so this is the combine step of the time scan.
__device__ __forceinline__ Hist hist_concat(const Hist& x, const Hist& y, float ny, float w2) {
  const float nx = x.n + ny;
  const float d = fmaf(-(nx - y.n), w2, x.kr - y.kr);  // scale of x minus scale of y
  const float e = exp2_fast(-fabsf(d));
  const bool keep = d >= 0.f;
  Hist r;
  r.A = keep ? fmaf(e, y.A, x.A) : fmaf(e, x.A, y.A);
  r.Bd = keep ? fmaf(e, y.Bd, x.Bd) : fmaf(e, x.Bd, y.Bd);
  r.kr = keep ? x.kr : y.kr;
  r.n = keep ? nx : y.n;
  return r;
}

// ---------------------------------------------------------------------------
// Cross-workgroup publication without fences: every published float travels
// in its own 64-bit word together with a 32-bit launch tag.  A word is valid
// for this launch iff its tag matches, so no flag/data ordering is needed.
// Agent-scope relaxed atomics keep the words coherent across the XCDs' L2s.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tagged_store(uint64_t* p, float x, uint32_t tag) {
  const uint64_t word = (uint64_t(tag) << 32) | uint64_t(__float_as_uint(x));
  __hip_atomic_store(p, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t tagged_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool tag_ok(uint64_t word, uint32_t tag) {
  return uint32_t(word >> 32) == tag;
}

__device__ __forceinline__ float tag_val(uint64_t word) {
  return __uint_as_float(uint32_t(word));
}

}  // namespace rwkv
