// C ABI of the WKV library: argument checks, plans, workspace sizing and
// launches.  Every check runs on the host before any HIP call; nothing here
// allocates, synchronises or prints.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "rwkv_wkv.h"
#include "wkv_internal.h"

#define RWKV_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip_error = 0;

// Largest element count accepted for any array (keeps byte sizes and 64-bit
// index arithmetic far from overflow).
constexpr int64_t kMaxElems = int64_t(1) << 56;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// out = a * b with a, b >= 0; false on overflow past kMaxElems.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kMaxElems / a) return false;
  *out = a * b;
  return true;
}

bool dims_ok(std::initializer_list<int64_t> dims, int64_t* numel) {
  int64_t n = 1;
  for (int64_t d : dims)
    if (!mul_ok(n, d, &n)) return false;
  *numel = n;
  return true;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return RWKV_OK;
  g_last_hip_error = int(e);
  return RWKV_ERR_HIP;
}

}  // namespace

// ------------------------------------------------------------ plan overrides

namespace rwkv {

namespace {

std::atomic<int> g_tune[kTuneKeys];
std::once_flag g_tune_once;

int env_int(const char* name) {
  const char* e = getenv(name);
  return e ? atoi(e) : 0;
}

// The environment's overrides, read once; values that no plan accepts are
// ignored (the built-in plan stays).
void tuning_from_env() {
  if (const char* e = getenv("RWKV_WKV4_TILE")) {
    int c = 0, l = 0, nw = 0;
    if (sscanf(e, "%d,%d,%d", &c, &l, &nw) == 3 && c > 0 && l > 0 && nw > 0)
      set_tuning(kTuneWkv4Tile, c * 10000 + l * 100 + nw);
  }
  if (const char* e = getenv("RWKV_WKV4_ORDER"))
    if (strcmp(e, "claim") == 0) set_tuning(kTuneWkv4Order, 1);
  set_tuning(kTuneWkv5Dv, env_int("RWKV_WKV5_DV"));
  set_tuning(kTuneWkv5Segs, env_int("RWKV_WKV5_SEGS"));
  set_tuning(kTuneWkv6Dv, env_int("RWKV_WKV6_DV"));
  set_tuning(kTuneWkv6Segs, env_int("RWKV_WKV6_SEGS"));
}

}  // namespace

bool set_tuning(int key, int value) {
  bool ok = false;
  switch (key) {
    case kTuneWkv4Tile: ok = value == 0 || wkv4_variant_exists(value); break;
    case kTuneWkv4Order: ok = value == 0 || value == 1; break;
    case kTuneWkv5Dv: ok = value == 0 || value == 16 || value == 32 || value == 64; break;
    case kTuneWkv6Dv: ok = value == 0 || value == 32 || value == 64; break;
    case kTuneWkv5Segs:
    case kTuneWkv6Segs: ok = value >= 0 && value <= 4096; break;
    case kTuneWkv4Spin: ok = value >= 0; break;
    default: ok = false;
  }
  if (ok) g_tune[key].store(value, std::memory_order_relaxed);
  return ok;
}

int tuning(int key) {
  std::call_once(g_tune_once, tuning_from_env);
  return key > 0 && key < kTuneKeys ? g_tune[key].load(std::memory_order_relaxed) : 0;
}

}  // namespace rwkv

RWKV_API int rwkv_set_tuning(int key, int value) {
  rwkv::tuning(key);  // the environment is read before the first explicit setting
  return rwkv::set_tuning(key, value) ? RWKV_OK : RWKV_ERR_UNSUPPORTED;
}

RWKV_API int rwkv_get_tuning(int key) { return rwkv::tuning(key); }

RWKV_API int rwkv_abi_version(void) { return RWKV_WKV_ABI_VERSION; }

RWKV_API const char* rwkv_status_str(int status) {
  switch (status) {
    case RWKV_OK: return "ok";
    case RWKV_ERR_NULLPTR: return "a required pointer is NULL";
    case RWKV_ERR_SHAPE: return "negative size or size overflow";
    case RWKV_ERR_UNSUPPORTED: return "shape not supported by this build";
    case RWKV_ERR_WORKSPACE: return "workspace missing or too small";
    case RWKV_ERR_ALIGN: return "pointer not 16-byte aligned";
    case RWKV_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

RWKV_API int rwkv_last_hip_error(void) { return g_last_hip_error; }

RWKV_API int rwkv_wkv4_workspace_error(const void* ws, size_t ws_bytes, uint32_t* err,
                                       hipStream_t stream) {
  if (!ws || !err) return RWKV_ERR_NULLPTR;
  if (ws_bytes < sizeof(uint32_t)) return RWKV_ERR_WORKSPACE;
  if (!aligned16(ws)) return RWKV_ERR_ALIGN;
  return hip_status(hipMemcpyAsync(err, ws, sizeof(uint32_t), hipMemcpyDefault, stream));
}

// ------------------------------------------------------------------ RWKV-4

RWKV_API size_t rwkv_wkv4_forward_workspace(int64_t B, int64_t T, int64_t C) {
  int64_t n;
  if (!dims_ok({B, T, C}, &n) || n == 0) return 0;
  rwkv::Wkv4Plan plan;
  if (!rwkv::wkv4_plan(B, T, C, &plan)) return 0;
  return plan.ws_bytes;
}

namespace {

int wkv4_forward_impl(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                      const float* k, const float* v, float* y, const float* a_in,
                      const float* b_in, const float* p_in, float* a_out, float* b_out,
                      float* p_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int64_t n;
  if (!dims_ok({B, T, C}, &n)) return RWKV_ERR_SHAPE;
  if (n == 0) return RWKV_OK;
  if (!w || !u || !k || !v || !y) return RWKV_ERR_NULLPTR;
  if (!aligned16(w) || !aligned16(u) || !aligned16(k) || !aligned16(v) || !aligned16(y))
    return RWKV_ERR_ALIGN;
  // A state triple is given whole or not at all.
  const int n_in = (a_in != nullptr) + (b_in != nullptr) + (p_in != nullptr);
  const int n_out = (a_out != nullptr) + (b_out != nullptr) + (p_out != nullptr);
  if ((n_in != 0 && n_in != 3) || (n_out != 0 && n_out != 3)) return RWKV_ERR_NULLPTR;
  if ((a_in && (!aligned16(a_in) || !aligned16(b_in) || !aligned16(p_in))) ||
      (a_out && (!aligned16(a_out) || !aligned16(b_out) || !aligned16(p_out))))
    return RWKV_ERR_ALIGN;
  rwkv::Wkv4Plan plan;
  if (!rwkv::wkv4_plan(B, T, C, &plan)) return RWKV_ERR_UNSUPPORTED;
  if (plan.ws_bytes > 0) {
    if (!ws || ws_bytes < plan.ws_bytes) return RWKV_ERR_WORKSPACE;
    if (!aligned16(ws)) return RWKV_ERR_ALIGN;
  }
  return hip_status(rwkv::wkv4_forward_launch(plan, B, T, C, w, u, k, v, y, ws, a_in, b_in,
                                              p_in, a_out, b_out, p_out, stream));
}

}  // namespace

RWKV_API int rwkv_wkv4_forward(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                               const float* k, const float* v, float* y, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  return wkv4_forward_impl(B, T, C, w, u, k, v, y, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, ws, ws_bytes, stream);
}

RWKV_API int rwkv_wkv4_forward_state(int64_t B, int64_t T, int64_t C, const float* w,
                                     const float* u, const float* k, const float* v, float* y,
                                     const float* a_in, const float* b_in, const float* p_in,
                                     float* a_out, float* b_out, float* p_out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  return wkv4_forward_impl(B, T, C, w, u, k, v, y, a_in, b_in, p_in, a_out, b_out, p_out, ws,
                           ws_bytes, stream);
}

RWKV_API int rwkv_wkv4_forward_noalloc(int64_t B, int64_t T, int64_t C, const float* w,
                                       const float* u, const float* k, const float* v, float* y,
                                       hipStream_t stream) {
  // Every check of the plain forward; a null workspace stops at the
  // workspace check (every plan needs one), after all the others.
  const int st = wkv4_forward_impl(B, T, C, w, u, k, v, y, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, 0, stream);
  if (st != RWKV_ERR_WORKSPACE) return st;
  rwkv::Wkv4Plan plan;
  if (!rwkv::wkv4_plan(B, T, C, &plan)) return RWKV_ERR_UNSUPPORTED;
  if (plan.ws_bytes > rwkv::noalloc_scratch_bytes()) return RWKV_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = rwkv::noalloc_scratch(&ws, stream);
  if (e != hipSuccess) return hip_status(e);
  return wkv4_forward_impl(B, T, C, w, u, k, v, y, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, ws, rwkv::noalloc_scratch_bytes(), stream);
}

RWKV_API int rwkv_wkv4_state_init(int64_t B, int64_t C, float* a, float* b, float* p,
                                  hipStream_t stream) {
  int64_t n;
  if (!dims_ok({B, C}, &n)) return RWKV_ERR_SHAPE;
  if (n == 0) return RWKV_OK;
  if (!a || !b || !p) return RWKV_ERR_NULLPTR;
  if (!aligned16(a) || !aligned16(b) || !aligned16(p)) return RWKV_ERR_ALIGN;
  return hip_status(rwkv::wkv4_state_init_launch(B, C, a, b, p, stream));
}

RWKV_API int rwkv_wkv4_step(int64_t B, int64_t C, float* a, float* b, float* p, const float* w,
                            const float* u, const float* k, const float* v, float* y,
                            hipStream_t stream) {
  int64_t n;
  if (!dims_ok({B, C}, &n)) return RWKV_ERR_SHAPE;
  if (n == 0) return RWKV_OK;
  if (!a || !b || !p || !w || !u || !k || !v || !y) return RWKV_ERR_NULLPTR;
  if (!aligned16(a) || !aligned16(b) || !aligned16(p) || !aligned16(w) || !aligned16(u) ||
      !aligned16(k) || !aligned16(v) || !aligned16(y))
    return RWKV_ERR_ALIGN;
  if (C >= (int64_t(1) << 31) || B >= (int64_t(1) << 31)) return RWKV_ERR_UNSUPPORTED;
  return hip_status(rwkv::wkv4_step_launch(B, C, a, b, p, w, u, k, v, y, stream));
}

RWKV_API size_t rwkv_wkv4_backward_workspace(int64_t B, int64_t T, int64_t C) {
  int64_t n;
  if (!dims_ok({B, T, C}, &n) || n == 0) return 0;
  rwkv::Wkv4BwdPlan plan;
  if (!rwkv::wkv4_backward_plan(B, T, C, &plan)) return 0;
  return plan.ws_bytes;
}

namespace {

int wkv4_backward_impl(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                       const float* k, const float* v, const float* gy, float* gw, float* gu,
                       float* gk, float* gv, void* ws, size_t ws_bytes, bool prefix_ready,
                       hipStream_t stream) {
  int64_t n;
  if (!dims_ok({B, T, C}, &n)) return RWKV_ERR_SHAPE;
  if (n == 0) return RWKV_OK;
  if (!w || !u || !k || !v || !gy || !gw || !gu || !gk || !gv) return RWKV_ERR_NULLPTR;
  if (!aligned16(w) || !aligned16(u) || !aligned16(k) || !aligned16(v) || !aligned16(gy) ||
      !aligned16(gw) || !aligned16(gu) || !aligned16(gk) || !aligned16(gv))
    return RWKV_ERR_ALIGN;
  rwkv::Wkv4BwdPlan plan;
  if (!rwkv::wkv4_backward_plan(B, T, C, &plan)) return RWKV_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < plan.ws_bytes) return RWKV_ERR_WORKSPACE;
  if (!aligned16(ws)) return RWKV_ERR_ALIGN;
  return hip_status(rwkv::wkv4_backward_launch(plan, B, T, C, w, u, k, v, gy, gw, gu, gk, gv, ws,
                                               prefix_ready, stream));
}

}  // namespace

RWKV_API int rwkv_wkv4_backward(int64_t B, int64_t T, int64_t C, const float* w, const float* u,
                                const float* k, const float* v, const float* gy, float* gw,
                                float* gu, float* gk, float* gv, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  return wkv4_backward_impl(B, T, C, w, u, k, v, gy, gw, gu, gk, gv, ws, ws_bytes, false,
                            stream);
}

RWKV_API int rwkv_wkv4_forward_train(int64_t B, int64_t T, int64_t C, const float* w,
                                     const float* u, const float* k, const float* v, float* y,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  int64_t n;
  if (!dims_ok({B, T, C}, &n)) return RWKV_ERR_SHAPE;
  if (n == 0) return RWKV_OK;
  if (!w || !u || !k || !v || !y) return RWKV_ERR_NULLPTR;
  if (!aligned16(w) || !aligned16(u) || !aligned16(k) || !aligned16(v) || !aligned16(y))
    return RWKV_ERR_ALIGN;
  rwkv::Wkv4BwdPlan plan;
  if (!rwkv::wkv4_backward_plan(B, T, C, &plan)) return RWKV_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < plan.ws_bytes) return RWKV_ERR_WORKSPACE;
  if (!aligned16(ws)) return RWKV_ERR_ALIGN;
  return hip_status(rwkv::wkv4_forward_train_launch(plan, T, C, w, u, k, v, y, ws, stream));
}

RWKV_API int rwkv_wkv4_backward_after_forward(int64_t B, int64_t T, int64_t C, const float* w,
                                              const float* u, const float* k, const float* v,
                                              const float* gy, float* gw, float* gu, float* gk,
                                              float* gv, void* ws, size_t ws_bytes,
                                              hipStream_t stream) {
  return wkv4_backward_impl(B, T, C, w, u, k, v, gy, gw, gu, gk, gv, ws, ws_bytes, true,
                            stream);
}

// ------------------------------------------------------------------- Eagle

RWKV_API size_t rwkv_wkv5_forward_workspace(int64_t B, int64_t T, int64_t H, int64_t D) {
  int64_t n;
  if (!dims_ok({B, T, H, D}, &n) || n == 0 || D != 64) return 0;
  return rwkv::wkv5_workspace_bytes(B, T, H, D);
}

namespace {

int wkv5_forward_impl(int64_t B, int64_t T, int64_t H, int64_t D, const uint16_t* r,
                      const uint16_t* k, const uint16_t* v, const float* w, const float* u,
                      float* o, const float* s_in, float* s_out, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  int64_t n;
  if (!dims_ok({B, T, H, D}, &n)) return RWKV_ERR_SHAPE;
  if (n == 0) return RWKV_OK;
  if (D != 64) return RWKV_ERR_UNSUPPORTED;
  if (T >= (int64_t(1) << 31) || B * H >= (int64_t(1) << 31) || H >= 65536)
    return RWKV_ERR_UNSUPPORTED;
  if (!r || !k || !v || !w || !u || !o) return RWKV_ERR_NULLPTR;
  if (!aligned16(r) || !aligned16(k) || !aligned16(v) || !aligned16(w) || !aligned16(u) ||
      !aligned16(o) || (s_in && !aligned16(s_in)) || (s_out && !aligned16(s_out)))
    return RWKV_ERR_ALIGN;
  const size_t need = rwkv::wkv5_workspace_bytes(B, T, H, D);
  if (need > 0) {
    if (!ws || ws_bytes < need) return RWKV_ERR_WORKSPACE;
    if (!aligned16(ws)) return RWKV_ERR_ALIGN;
  }
  return hip_status(
      rwkv::wkv5_forward_launch(B, T, H, D, r, k, v, w, u, o, ws, s_in, s_out, stream));
}

}  // namespace

RWKV_API int rwkv_wkv5_forward(int64_t B, int64_t T, int64_t H, int64_t D, const uint16_t* r,
                               const uint16_t* k, const uint16_t* v, const float* w,
                               const float* u, float* o, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  return wkv5_forward_impl(B, T, H, D, r, k, v, w, u, o, nullptr, nullptr, ws, ws_bytes,
                           stream);
}

RWKV_API int rwkv_wkv5_forward_state(int64_t B, int64_t T, int64_t H, int64_t D,
                                     const uint16_t* r, const uint16_t* k, const uint16_t* v,
                                     const float* w, const float* u, float* o,
                                     const float* s_in, float* s_out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  return wkv5_forward_impl(B, T, H, D, r, k, v, w, u, o, s_in, s_out, ws, ws_bytes, stream);
}

RWKV_API int rwkv_wkv5_step(int64_t B, int64_t H, int64_t D, float* s, const uint16_t* r,
                            const uint16_t* k, const uint16_t* v, const float* w,
                            const float* u, float* o, hipStream_t stream) {
  int64_t n;
  if (!dims_ok({B, H, D}, &n)) return RWKV_ERR_SHAPE;
  if (n == 0) return RWKV_OK;
  if (D != 64) return RWKV_ERR_UNSUPPORTED;
  if (B * H >= (int64_t(1) << 31)) return RWKV_ERR_UNSUPPORTED;
  if (!s || !r || !k || !v || !w || !u || !o) return RWKV_ERR_NULLPTR;
  if (!aligned16(s) || !aligned16(r) || !aligned16(k) || !aligned16(v) || !aligned16(w) ||
      !aligned16(u) || !aligned16(o))
    return RWKV_ERR_ALIGN;
  return hip_status(rwkv::wkv5_step_launch(B, H, s, r, k, v, w, u, o, stream));
}

// ------------------------------------------------------------------- Finch

RWKV_API size_t rwkv_wkv6_forward_workspace(int64_t B, int64_t T, int64_t H, int64_t D) {
  int64_t n;
  if (!dims_ok({B, T, H, D}, &n) || n == 0 || D != 64) return 0;
  return rwkv::wkv6_workspace_bytes(B, T, H);
}

RWKV_API int rwkv_wkv6_forward(int64_t B, int64_t T, int64_t H, int64_t D, const uint16_t* r,
                               const uint16_t* k, const uint16_t* v, const float* w,
                               const float* u, float* o, const float* s_in, float* s_out,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  int64_t n;
  if (!dims_ok({B, T, H, D}, &n)) return RWKV_ERR_SHAPE;
  if (n == 0) return RWKV_OK;
  if (D != 64) return RWKV_ERR_UNSUPPORTED;
  if (T >= (int64_t(1) << 31) || B * H >= (int64_t(1) << 31) || H >= 65536)
    return RWKV_ERR_UNSUPPORTED;
  if (!r || !k || !v || !w || !u || !o) return RWKV_ERR_NULLPTR;
  if (!aligned16(r) || !aligned16(k) || !aligned16(v) || !aligned16(w) || !aligned16(u) ||
      !aligned16(o) || (s_in && !aligned16(s_in)) || (s_out && !aligned16(s_out)))
    return RWKV_ERR_ALIGN;
  const size_t need = rwkv::wkv6_workspace_bytes(B, T, H);
  if (need > 0) {
    if (!ws || ws_bytes < need) return RWKV_ERR_WORKSPACE;
    if (!aligned16(ws)) return RWKV_ERR_ALIGN;
  }
  return hip_status(
      rwkv::wkv6_forward_launch(B, T, H, r, k, v, w, u, o, s_in, s_out, ws, stream));
}

RWKV_API int rwkv_wkv6_step(int64_t B, int64_t H, int64_t D, float* s, const uint16_t* r,
                            const uint16_t* k, const uint16_t* v, const float* w,
                            const float* u, float* o, hipStream_t stream) {
  int64_t n;
  if (!dims_ok({B, H, D}, &n)) return RWKV_ERR_SHAPE;
  if (n == 0) return RWKV_OK;
  if (D != 64) return RWKV_ERR_UNSUPPORTED;
  if (B * H >= (int64_t(1) << 31)) return RWKV_ERR_UNSUPPORTED;
  if (!s || !r || !k || !v || !w || !u || !o) return RWKV_ERR_NULLPTR;
  if (!aligned16(s) || !aligned16(r) || !aligned16(k) || !aligned16(v) || !aligned16(w) ||
      !aligned16(u) || !aligned16(o))
    return RWKV_ERR_ALIGN;
  return hip_status(rwkv::wkv6_step_launch(B, H, s, r, k, v, w, u, o, stream));
}
