// Pieces shared by the Eagle and Finch matrix-state kernels on gfx950: head
// and chunk sizes, bf16 helpers, one thread's share of a chunk's r, k, v and
// the bf16 MFMA used for every chunk product.
#pragma once

#include "wkv_device.h"

namespace rwkv {
namespace eagle {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kD = 64;        // head size
constexpr int kL = 64;        // chunk length
constexpr int kPad = 72;      // LDS row length in bf16 (144 bytes: 16-byte aligned rows)

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(uint32_t(x) << 16);
}

// float -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }

// Chunks stream through buffer resources spanning one chunk's rows of a
// [B, T, H, kD] tensor: a lane's offset within the chunk is computed once,
// no 64-bit address arithmetic is spent per access, bytes past the last row
// of the sequence read as zero and stores there are dropped by the hardware.
// The span is at most 64 rows of H kD floats, below 2^31 bytes for
// H < 2^17 (the callers reject larger H).  Measured at B=4 T=4096 H=32:
// loads are faster with the default cache policy (the non-temporal hint cost
// the Eagle forward about 8%), o stores with the non-temporal one (Eagle
// 93 -> 80 us, Finch 197 -> 187 us).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit access, gfx9 family
constexpr int kLoadAux = 0;
constexpr int kStoreAux = 2;            // non-temporal

// Resource over rows t0 .. t0 + n_tok - 1 of head h (element size `esz`);
// with live = false it spans nothing, so every access through it is dropped
// (reads give zero) without touching memory.
__device__ __forceinline__ Rsrc chunk_rsrc(const void* base, int t0, int T, int H, int b, int h,
                                           int esz, bool live = true) {
  const size_t e0 = ((size_t(b) * T + t0) * H + h) * kD;
  const int n_tok = min(kL, T - t0);
  const uint32_t bytes = live ? uint32_t(((n_tok - 1) * H + 1) * kD * esz) : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(base)) + e0 * esz, 0, int(bytes), kRsrcWord3);
}

__device__ __forceinline__ uint4 load16(Rsrc rs, uint32_t voff) {
  typedef int iv4 __attribute__((ext_vector_type(4)));
  const iv4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, kLoadAux);
  return uint4{uint32_t(t.x), uint32_t(t.y), uint32_t(t.z), uint32_t(t.w)};
}

// One chunk's raw inputs for this thread: token tau = tid/4, dims 16*(tid%4)
// of r and k, and DV/4 value dims of this workgroup's slice (16, 8 or 4);
// zeros past T.
struct ChunkRegs {
  uint4 r0, r1, k0, k1, v0, v1;  // v1: the second half of 16 value dims (DV = 64)
};

// WITH_R = false (segment states) skips r.  live = false issues the same
// loads through empty resources (zeros, no memory traffic).
template <int DV, bool WITH_R = true>
__device__ __forceinline__ void load_chunk(ChunkRegs& x, int t0, int T, int H, int b, int h,
                                           int j0, const uint16_t* __restrict__ r,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v, bool live = true) {
  const int tid = threadIdx.x;
  const int tau = tid >> 2, q4 = tid & 3;
  const uint32_t row = uint32_t(tau * H * kD);
  const Rsrc rk = chunk_rsrc(k, t0, T, H, b, h, 2, live);
  const Rsrc rv = chunk_rsrc(v, t0, T, H, b, h, 2, live);
  const uint32_t off = (row + 16 * q4) * 2;
  if constexpr (WITH_R) {
    const Rsrc rr = chunk_rsrc(r, t0, T, H, b, h, 2, live);
    x.r0 = load16(rr, off);
    x.r1 = load16(rr, off + 16);
  } else {
    x.r0 = x.r1 = uint4{0u, 0u, 0u, 0u};
  }
  x.k0 = load16(rk, off);
  x.k1 = load16(rk, off + 16);
  x.v1 = uint4{0u, 0u, 0u, 0u};
  if constexpr (DV == 64) {
    x.v0 = load16(rv, off);
    x.v1 = load16(rv, off + 16);
  } else if constexpr (DV == 32) {
    x.v0 = load16(rv, (row + j0 + 8 * q4) * 2);
  } else {
    typedef int iv2 __attribute__((ext_vector_type(2)));
    const iv2 t = __builtin_amdgcn_raw_buffer_load_b64(rv, (row + j0 + 4 * q4) * 2, 0,
                                                       kLoadAux);
    x.v0 = uint4{uint32_t(t.x), uint32_t(t.y), 0u, 0u};
  }
}

__device__ __forceinline__ float lo_half(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_half(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// MFMA operands of a product summed over tokens (K = sigma), read from a
// row-major [sigma][column] tile with gfx950's LDS transpose load: within each
// 16-lane group, lane r addresses 4 elements of row k0 + r/4, columns
// c0 + 4 (r % 4) .. + 3, and lane i receives column c0 + i of rows k0 .. k0 + 3
// (lane layout confirmed by an in-bounds probe).  Two such loads give an
// 8-element operand; K is ordered per 16-lane group g as sigma =
// s0 + 4g + 0..3, then s0 + 16 + 4g + 0..3, which is the order of the masked
// score tiles held in registers (the accumulator rows of two 16-token
// blocks), so every product over sigma uses it.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4i16 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<__bf16*>(p)));
}

// Operand for tokens s0 .. s0 + 31 (in the order above) and columns
// c0 .. c0 + 15 of a [sigma][kPad] tile.
__device__ __forceinline__ bf16x8 sigma_operand(const __bf16 (*tile)[kPad], int s0, int c0,
                                                int lane) {
  const int g = lane >> 4, r = lane & 15;
  const __bf16* p = &tile[s0 + 4 * g + (r >> 2)][c0 + 4 * (r & 3)];
  const v4i16 lo = lds_read_tr(p);
  const v4i16 hi = lds_read_tr(p + 16 * kPad);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ floatx4 mfma(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace eagle
}  // namespace rwkv
