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
// RWKV-4 state arithmetic in the base-2 domain.
//
// A lane's history is (A, Bd, p): numerator and denominator sums scaled by
// 2^p, with k, w, u pre-multiplied by log2(e).  Each update keeps the larger
// of the two exponents as the new scale, so one of the two terms is taken at
// factor 1 and a single exp2 of a non-positive number is needed.
// ---------------------------------------------------------------------------
struct Hist {
  float A, Bd, p;
};

__device__ __forceinline__ Hist hist_empty() { return Hist{0.f, 0.f, kEmptyP}; }

// Advance the history by one token: decay by 2^-w2, add 2^k2 * (v, 1).
__device__ __forceinline__ void hist_push(Hist& h, float k2, float v, float w2) {
  const float pd = h.p - w2;
  const float d = pd - k2;
  const float e = exp2_fast(-fabsf(d));
  const bool keep = d >= 0.f;  // history dominates: it stays at factor 1
  const float a_one = keep ? h.A : v;
  const float a_scl = keep ? v : h.A;
  const float b_one = keep ? h.Bd : 1.f;
  const float b_scl = keep ? 1.f : h.Bd;
  h.A = fmaf(e, a_scl, a_one);
  h.Bd = fmaf(e, b_scl, b_one);
  h.p = keep ? pd : k2;
}

// Output for the current token: (history + 2^(u2+k2) v) / (history + 2^(u2+k2)).
__device__ __forceinline__ float hist_read(const Hist& h, float k2, float v, float u2) {
  const float cur = u2 + k2;
  const float d = h.p - cur;
  const float e = exp2_fast(-fabsf(d));
  const bool keep = d >= 0.f;
  const float num = keep ? fmaf(e, v, h.A) : fmaf(e, h.A, v);
  const float den = keep ? (h.Bd + e) : fmaf(e, h.Bd, 1.f);
  return num * rcp_fast(den);
}

// Concatenate histories: `x` covers an earlier stretch, `y` the `ny` tokens
// right after it (y was accumulated from an empty history).  Decay and sum
// are associative, so this is the combine step of the time scan.  ny * w2 is
// one multiply, never a repeated subtraction.
__device__ __forceinline__ Hist hist_concat(const Hist& x, const Hist& y, float ny_w2) {
  const float px = x.p - ny_w2;
  const float d = px - y.p;
  const float e = exp2_fast(-fabsf(d));
  const bool keep = d >= 0.f;
  Hist r;
  r.A = keep ? fmaf(e, y.A, x.A) : fmaf(e, x.A, y.A);
  r.Bd = keep ? fmaf(e, y.Bd, x.Bd) : fmaf(e, x.Bd, y.Bd);
  r.p = keep ? px : y.p;
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
