// Copy-peak kernels for the benchmark (not part of the operator library):
// elementwise sums whose traffic is that of a forward with no dependencies
// between elements, loads and stores non-temporal, so that their rate on the
// same box and the same buffers is the practical ceiling the forward's HBM
// rate is compared against.  add_copy: y = a + b over float32 arrays (the
// RWKV-4 forward's 12 bytes per element); mix_copy: three bfloat16 inputs
// (and optionally a float32 one) into a float32 output (the Eagle and Finch
// forwards' 10 and 14 bytes); three_two_copy: three float32 arrays into two
// (the RWKV-4 backward's 20 bytes).
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void add_copy(size_t n4, const f4* __restrict__ a,
                                                const f4* __restrict__ b, f4* __restrict__ y) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) {
    const f4 x = __builtin_nontemporal_load(a + i);
    const f4 z = __builtin_nontemporal_load(b + i);
    __builtin_nontemporal_store(x + z, y + i);
  }
}

// The matrix-state forwards' traffic: three bfloat16 inputs (and, for a
// per-token decay, a float32 one) read and one float32 output written per
// element, 8 elements per thread.
typedef unsigned short us8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf(unsigned short x) { return __uint_as_float(unsigned(x) << 16); }

template <bool WITH_W>
__global__ __launch_bounds__(256) void mix_copy(size_t n8, const us8* __restrict__ r,
                                                const us8* __restrict__ k,
                                                const us8* __restrict__ v,
                                                const f4* __restrict__ w, f4* __restrict__ o) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n8) {
    const us8 a = __builtin_nontemporal_load(r + i);
    const us8 b = __builtin_nontemporal_load(k + i);
    const us8 c = __builtin_nontemporal_load(v + i);
    f4 lo = {bf(a[0]) + bf(b[0]) + bf(c[0]), bf(a[1]) + bf(b[1]) + bf(c[1]),
             bf(a[2]) + bf(b[2]) + bf(c[2]), bf(a[3]) + bf(b[3]) + bf(c[3])};
    f4 hi = {bf(a[4]) + bf(b[4]) + bf(c[4]), bf(a[5]) + bf(b[5]) + bf(c[5]),
             bf(a[6]) + bf(b[6]) + bf(c[6]), bf(a[7]) + bf(b[7]) + bf(c[7])};
    if (WITH_W) {
      lo += __builtin_nontemporal_load(w + 2 * i);
      hi += __builtin_nontemporal_load(w + 2 * i + 1);
    }
    __builtin_nontemporal_store(lo, o + 2 * i);
    __builtin_nontemporal_store(hi, o + 2 * i + 1);
  }
}

// The RWKV-4 backward's traffic: three float32 arrays read, two written.
__global__ __launch_bounds__(256) void three_two_copy(size_t n4, const f4* __restrict__ a,
                                                      const f4* __restrict__ b,
                                                      const f4* __restrict__ c,
                                                      f4* __restrict__ y, f4* __restrict__ z) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) {
    const f4 x0 = __builtin_nontemporal_load(a + i);
    const f4 x1 = __builtin_nontemporal_load(b + i);
    const f4 x2 = __builtin_nontemporal_load(c + i);
    __builtin_nontemporal_store(x0 + x1, y + i);
    __builtin_nontemporal_store(x1 + x2, z + i);
  }
}

}  // namespace

// y[i] = a[i] + b[i], z[i] = b[i] + c[i] for i < n, float32: 20 bytes per
// element, the traffic of the RWKV-4 backward (k, v, gy read; gk, gv
// written).  n must be a multiple of 4 and every pointer 16-byte aligned
// (else -1).  Returns 0 or the launch's hipError_t.
extern "C" __attribute__((visibility("default"))) int wkv_bench_three_two_copy(
    const float* a, const float* b, const float* c, float* y, float* z, size_t n,
    hipStream_t stream) {
  if (n % 4 != 0 || (reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                     reinterpret_cast<uintptr_t>(c) | reinterpret_cast<uintptr_t>(y) |
                     reinterpret_cast<uintptr_t>(z)) % 16 != 0)
    return -1;
  const size_t n4 = n / 4;
  if (n4 == 0) return 0;
  const size_t blocks = (n4 + 255) / 256;
  if (blocks >= (size_t(1) << 31)) return -1;
  hipLaunchKernelGGL(three_two_copy, dim3(unsigned(blocks)), dim3(256), 0, stream, n4,
                     reinterpret_cast<const f4*>(a), reinterpret_cast<const f4*>(b),
                     reinterpret_cast<const f4*>(c), reinterpret_cast<f4*>(y),
                     reinterpret_cast<f4*>(z));
  return int(hipGetLastError());
}

// o[i] = r[i] + k[i] + v[i] (+ w[i] when w is not null) for i < n, with r, k,
// v bfloat16 bit patterns and w, o float32: 10 (14 with w) bytes per
// element, the traffic of the Eagle (Finch) forward.  n must be a multiple
// of 8 and every pointer 16-byte aligned (else -1).  Returns 0 or the
// launch's hipError_t.
extern "C" __attribute__((visibility("default"))) int wkv_bench_mix_copy(
    const uint16_t* r, const uint16_t* k, const uint16_t* v, const float* w, float* o, size_t n,
    hipStream_t stream) {
  if (n % 8 != 0 || (reinterpret_cast<uintptr_t>(r) | reinterpret_cast<uintptr_t>(k) |
                     reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(w) |
                     reinterpret_cast<uintptr_t>(o)) % 16 != 0)
    return -1;
  const size_t n8 = n / 8;
  if (n8 == 0) return 0;
  const size_t blocks = (n8 + 255) / 256;
  if (blocks >= (size_t(1) << 31)) return -1;
  if (w)
    hipLaunchKernelGGL(mix_copy<true>, dim3(unsigned(blocks)), dim3(256), 0, stream, n8,
                       reinterpret_cast<const us8*>(r), reinterpret_cast<const us8*>(k),
                       reinterpret_cast<const us8*>(v), reinterpret_cast<const f4*>(w),
                       reinterpret_cast<f4*>(o));
  else
    hipLaunchKernelGGL(mix_copy<false>, dim3(unsigned(blocks)), dim3(256), 0, stream, n8,
                       reinterpret_cast<const us8*>(r), reinterpret_cast<const us8*>(k),
                       reinterpret_cast<const us8*>(v), nullptr, reinterpret_cast<f4*>(o));
  return int(hipGetLastError());
}

// y[i] = a[i] + b[i] for i < n.  n must be a multiple of 4 and every
// pointer 16-byte aligned (else -1); n = 0 launches nothing.  Returns 0 or
// the launch's hipError_t.
extern "C" __attribute__((visibility("default"))) int wkv_bench_add_copy(
    const float* a, const float* b, float* y, size_t n, hipStream_t stream) {
  if (n % 4 != 0 || (reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                     reinterpret_cast<uintptr_t>(y)) % 16 != 0)
    return -1;
  const size_t n4 = n / 4;
  if (n4 == 0) return 0;
  const size_t blocks = (n4 + 255) / 256;
  if (blocks >= (size_t(1) << 31)) return -1;
  hipLaunchKernelGGL(add_copy, dim3(unsigned(blocks)), dim3(256), 0, stream, n4,
                     reinterpret_cast<const f4*>(a), reinterpret_cast<const f4*>(b),
                     reinterpret_cast<f4*>(y));
  return int(hipGetLastError());
}
