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

// One chunk's raw inputs for this thread: token tau = tid/4, dims 16*(tid%4)
// of r and k, and DV/4 value dims of this workgroup's slice (16, 8 or 4).
struct ChunkRegs {
  uint4 r0, r1, k0, k1, v0, v1;  // v1: the second half of 16 value dims (DV = 64)
};

template <int DV>
__device__ __forceinline__ void load_chunk(ChunkRegs& x, int t0, int T, int H, int b, int h,
                                           int j0, const uint16_t* __restrict__ r,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v) {
  const int tid = threadIdx.x;
  const int tau = tid >> 2, q4 = tid & 3;
  if (t0 + tau < T) {
    const size_t off = ((size_t(b) * T + t0 + tau) * H + h) * kD;
    const uint4* rp = reinterpret_cast<const uint4*>(r + off + 16 * q4);
    const uint4* kp = reinterpret_cast<const uint4*>(k + off + 16 * q4);
    x.r0 = rp[0];
    x.r1 = rp[1];
    x.k0 = kp[0];
    x.k1 = kp[1];
    x.v1 = uint4{0u, 0u, 0u, 0u};
    if constexpr (DV == 64) {
      x.v0 = *reinterpret_cast<const uint4*>(v + off + 16 * q4);
      x.v1 = *reinterpret_cast<const uint4*>(v + off + 16 * q4 + 8);
    } else if constexpr (DV == 32) {
      x.v0 = *reinterpret_cast<const uint4*>(v + off + j0 + 8 * q4);
    } else {
      const uint2 t = *reinterpret_cast<const uint2*>(v + off + j0 + 4 * q4);
      x.v0 = uint4{t.x, t.y, 0u, 0u};
    }
  } else {
    x.r0 = x.r1 = x.k0 = x.k1 = x.v0 = x.v1 = uint4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ float lo_half(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_half(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ floatx4 mfma(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace eagle
}  // namespace rwkv
