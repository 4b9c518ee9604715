// Eagle (RWKV-5) matrix-state WKV kernels for gfx950.
//
// What is computed: [Eagle-Finch] "RWKV-5 Eagle and RWKV-6 Finch" (ql.gl
// blog), section "Eagle: extending vector memory to matrix memory":
//   s' = diag(w) s + k^T v,   wkv' = s + diag(u) k^T v,
// with the receptance reading wkv' like a query.  Per (batch, head) the state
// s is D x D, indexed [key i][value j]; diag(w) scales key rows.
#include "wkv_device.h"
#include "wkv_internal.h"

namespace rwkv {

namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(uint32_t(x) << 16);
}

// Token-by-token recurrence: one workgroup per (batch, head), one lane per
// value column j holding the state column s[:, j] (64 floats) in registers.
// Exact float32 arithmetic on the bf16 inputs.
__global__ __launch_bounds__(64) void wkv5_fwd_recurrent64(
    int T, int H, const uint16_t* __restrict__ r, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ w,
    const float* __restrict__ u, float* __restrict__ o) {
  constexpr int D = 64;
  __shared__ float s_r[D], s_k[D], s_w[D], s_u[D];
  const int bh = blockIdx.x;
  const int b = bh / H;
  const int h = bh - b * H;
  const int j = threadIdx.x;
  s_w[j] = w[h * D + j];
  s_u[j] = u[h * D + j];
  float S[D];
#pragma unroll
  for (int i = 0; i < D; ++i) S[i] = 0.f;
  for (int t = 0; t < T; ++t) {
    const size_t off = ((size_t(b) * T + t) * H + h) * D;
    const float vj = bf16_to_f32(v[off + j]);
    s_r[j] = bf16_to_f32(r[off + j]);
    s_k[j] = bf16_to_f32(k[off + j]);
    __syncthreads();
    float acc = 0.f, beta = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const float ri = s_r[i], ki = s_k[i];
      acc = fmaf(ri, S[i], acc);
      beta = fmaf(ri * s_u[i], ki, beta);
      S[i] = fmaf(s_w[i], S[i], ki * vj);
    }
    o[off + j] = fmaf(beta, vj, acc);
    __syncthreads();
  }
}

}  // namespace

size_t wkv5_workspace_bytes(int64_t, int64_t, int64_t, int64_t) { return 0; }

hipError_t wkv5_forward_launch(int64_t B, int64_t T, int64_t H, int64_t D,
                               const uint16_t* r, const uint16_t* k, const uint16_t* v,
                               const float* w, const float* u, float* o, void* ws,
                               hipStream_t stream) {
  (void)D;
  (void)ws;
  hipLaunchKernelGGL(wkv5_fwd_recurrent64, dim3(unsigned(B * H)), dim3(64), 0, stream, int(T),
                     int(H), r, k, v, w, u, o);
  return hipGetLastError();
}

}  // namespace rwkv
