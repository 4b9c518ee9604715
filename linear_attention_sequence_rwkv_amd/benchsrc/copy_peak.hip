// Copy-peak kernel for the benchmark (not part of the operator library):
// y = a + b over float32 arrays, one 16-byte vector per thread, loads and
// stores non-temporal.  It moves the RWKV-4 forward's 12 bytes per element
// (read two arrays, write one) with no dependencies between elements, so
// its rate on the same box and the same buffers is the practical ceiling
// the forward's HBM rate is compared against.
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

}  // namespace

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
