// Scratch of the RWKV-4 forward for callers that cannot allocate
// (rwkv_wkv4_forward_noalloc): the look-back workspace is a file-scope device
// array instead of a caller's buffer.
//
// The array is the library's own, one copy per GPU for the life of the
// process.  Its device address is taken once per device with
// hipGetSymbolAddress (in host code the array's name is only a host-side
// stand-in) and the array is zero-filled by a kernel on that first call's
// stream; after that the forward's tagged words keep it valid for any later
// call of any shape, so nothing is cleared between calls.  The forward's tags
// come from a 32-bit epoch that advances once per call, so the host counts
// the calls per device and zero-fills the array again every 2^30 calls, long
// before the epoch could wrap.  Calls that overlap on one GPU (other
// streams, other threads) share the array and race.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "wkv_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void zero_scratch(uint4* __restrict__ p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

constexpr int kMaxDevices = 64;
constexpr uint64_t kRezeroEvery = uint64_t(1) << 30;

struct DeviceScratch {
  void* ptr = nullptr;         // device address of `scratch` on this device
  uint64_t calls = 0;          // calls since the last zero fill
  bool zeroed = false;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

// The current device's copy of the array, zero-filled on `stream` when it
// is new or its call count has come round.  Returns a HIP error.
hipError_t scratch_for_call(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& d = g_dev[dev];
  if (!d.ptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    d.ptr = p;
  }
  if (!d.zeroed || d.calls >= kRezeroEvery) {
    const size_t n = kScratchBytes / sizeof(uint4);
    hipLaunchKernelGGL(zero_scratch, dim3(1024), dim3(256), 0, stream, static_cast<uint4*>(d.ptr),
                       n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // A fill recorded into a graph that is being captured has not run yet:
    // fill again at the next call made outside the capture.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    d.zeroed = hipStreamIsCapturing(stream, &cs) == hipSuccess &&
               cs == hipStreamCaptureStatusNone;
    d.calls = 0;
  }
  ++d.calls;
  *out = d.ptr;
  return hipSuccess;
}

}  // namespace

namespace rwkv {

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** out, hipStream_t stream) { return scratch_for_call(out, stream); }

}  // namespace rwkv
