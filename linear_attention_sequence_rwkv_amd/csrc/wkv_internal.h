// Host-side declarations shared between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rwkv {

// ----- Plan overrides (tests and sweeps) -----
//
// Each key holds 0 (the built-in plan) or an override; the values start from
// the environment (RWKV_WKV4_TILE="cpl,L,NW", RWKV_WKV4_ORDER=claim,
// RWKV_WKV5_DV, RWKV_WKV5_SEGS, RWKV_WKV6_DV, RWKV_WKV6_SEGS), read once, and
// rwkv_set_tuning changes them.  They select other tile shapes, value slices
// and time segments, and so change the workspace sizes.
enum TuneKey : int {
  kTuneWkv4Tile = 1,   // [cb * 100000 +] cpl * 10000 + L * 100 + NW of a compiled forward shape
  kTuneWkv4Order = 2,  // 1: claimed tiles even where the grid is resident
  kTuneWkv5Dv = 3,     // value columns per Eagle workgroup: 16, 32 or 64
  kTuneWkv5Segs = 4,   // Eagle time segments (before the clamp to >= 4 chunks each)
  kTuneWkv6Dv = 5,     // value columns per Finch workgroup: 32 or 64
  kTuneWkv6Segs = 6,   // Finch time segments
  kTuneWkv4Spin = 7,   // polls of an RWKV-4 look-back before it gives up (0: the default)
  kTuneKeys = 8
};
int tuning(int key);
bool set_tuning(int key, int value);
// Whether the forward has a compiled tile shape with this code.
bool wkv4_variant_exists(int code);

// Longest sequence of one RWKV-4 call: decay counts are held as floats,
// exact for integers up to 2^24.  Longer sequences are cut and chained
// through the state entry points.
constexpr int64_t kWkv4MaxT = (int64_t(1) << 24) - 64;

// ----- RWKV-4 forward: single-pass tiled scan with decoupled look-back -----
//
// A channel block is 64*CPL channels (CPL per lane); a tile is L tokens per
// wave x NW waves stacked along time, so a workgroup covers TILE = L * NW
// tokens of one block.  Workspace: a header (error word), one 64-bit tagged
// ticket counter per (batch, block) every kWkv4CounterStride bytes, then per
// (tile, block) two published histories (aggregate, inclusive) of 4 tagged
// 64-bit words per channel each.
struct Wkv4Plan {
  int cb;        // channel blocks per workgroup (each with its own tiles)
  int cpl;       // channels per lane (vector width of the loads)
  int L;         // tokens per wave
  int NW;        // waves per workgroup
  int64_t tile;  // L * NW
  int64_t n_tiles;
  int64_t n_cblk;  // ceil(C / (64 * cpl))
  int64_t groups;  // B * n_cblk
  size_t slots_offset;
  size_t ws_bytes;
};

constexpr size_t kWkv4HeaderBytes = 128;
constexpr size_t kWkv4CounterStride = 128;  // one counter per 128-byte line

// Polls an RWKV-4 look-back (forward or reverse) makes before it gives up,
// raises error bit 0 and writes NaN: the kTuneWkv4Spin override, else 2^24.
uint32_t wkv4_spin_limit();

// Whether the passes that read k and v twice (the backward's prefix and
// reverse passes, the training forward and the backward after it) load them
// on the default cache policy, so that the second read meets them in the
// MALL, instead of non-temporally: k and v together at most kKeepRowBytes.
// Backward at 8x1024x768: 53.0 -> 45.1 us on one input set, 54.7 -> 52.1 us
// over six rotated sets; training pair: 57.2 -> 47.9 and 58.9 -> 58.6 us
// (with the training forward left non-temporal, 62.0 over six sets).  At
// 1x65536x5120 (2.7 GB) the default policy cost 1.3%.
constexpr int64_t kKeepRowBytes = int64_t(128) << 20;
bool wkv4_keep_rows(const Wkv4Plan& pl, int64_t T, int64_t C);

// Plan for a shape; honours the kTuneWkv4Tile override.  Returns false if
// the shape cannot be planned (T > kWkv4MaxT, or too large for 32-bit
// tickets and offsets).
bool wkv4_plan(int64_t B, int64_t T, int64_t C, Wkv4Plan* plan);
// The same for a given tile shape.
bool wkv4_plan_fixed(int64_t B, int64_t T, int64_t C, int cpl, int L, int NW, Wkv4Plan* plan);
// Channel blocks per workgroup (1 or 2) for the 1 x 32 x 4 tiles of a shape.
int wkv4_grouped_cb(int64_t B, int64_t T, int64_t C);

// The forward scan without output rows: publishes every tile's inclusive
// history in the workspace (plan: one channel per lane, 32 x 4 tiles) and,
// in `mids` (tagged words, 4 x 64 per tile and channel block), the inclusive
// history after the first 64 tokens of each tile.
hipError_t wkv4_prefix_launch(const Wkv4Plan& plan, int64_t T, int64_t C, const float* w,
                              const float* u, const float* k, const float* v, void* ws,
                              void* mids, hipStream_t stream);

// The forward with outputs, also publishing the prefix pass's histories
// (tile shape 1 x 32 x 4 only).
hipError_t wkv4_forward_tape_launch(const Wkv4Plan& plan, int64_t T, int64_t C, const float* w,
                                   const float* u, const float* k, const float* v, float* y,
                                   void* ws, void* mids, hipStream_t stream);

// a/b/p_in: optional history before the first token; a/b/p_out: optional
// state after the last token (both [B, C], step-API form; may be null).
hipError_t wkv4_forward_launch(const Wkv4Plan& plan, int64_t B, int64_t T, int64_t C,
                               const float* w, const float* u, const float* k,
                               const float* v, float* y, void* ws, const float* a_in,
                               const float* b_in, const float* p_in, float* a_out,
                               float* b_out, float* p_out, hipStream_t stream);

hipError_t wkv4_state_init_launch(int64_t B, int64_t C, float* a, float* b, float* p,
                                  hipStream_t stream);

hipError_t wkv4_step_launch(int64_t B, int64_t C, float* a, float* b, float* p,
                            const float* w, const float* u, const float* k,
                            const float* v, float* y, hipStream_t stream);

// The forward's workspace for callers that cannot allocate: a file-scope
// device array of noalloc_scratch_bytes() per GPU, zero-filled on `stream`
// at its first use on the current device (and again every 2^30 calls).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out, hipStream_t stream);

// ----- RWKV-4 backward -----
//
// Workspace: the prefix pass's forward workspace (its header and counters
// serve both passes), then the reverse scan's published histories (6
// fields, aggregate and inclusive, per tile and channel), then the gw and gu
// partial sums per (tile, sequence, channel) as tagged words.
struct Wkv4BwdPlan {
  Wkv4Plan fwd;      // prefix pass: 128-token tiles
  int64_t rev_tiles;  // reverse pass: 64-token tiles, same channel blocks
  size_t mid_offset;  // the prefix pass's mid-tile histories
  size_t rev_slots_offset;
  size_t part_offset;
  int64_t part_rows;  // rev_tiles * B
  size_t ws_bytes;
};

bool wkv4_backward_plan(int64_t B, int64_t T, int64_t C, Wkv4BwdPlan* plan);

// prefix_ready: the workspace already holds the prefix pass's histories,
// left there by wkv4_forward_train_launch over the same inputs.
hipError_t wkv4_backward_launch(const Wkv4BwdPlan& plan, int64_t B, int64_t T, int64_t C,
                                const float* w, const float* u, const float* k,
                                const float* v, const float* gy, float* gw, float* gu,
                                float* gk, float* gv, void* ws, bool prefix_ready,
                                hipStream_t stream);

// The forward with outputs over a backward workspace, publishing the same
// histories as the backward's prefix pass (with the prefix pass's tiles).
hipError_t wkv4_forward_train_launch(const Wkv4BwdPlan& plan, int64_t T, int64_t C,
                                     const float* w, const float* u, const float* k,
                                     const float* v, float* y, void* ws, hipStream_t stream);

// ----- Eagle (RWKV-5) forward -----
size_t wkv5_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t D);

// s_in / s_out: optional [B, H, D, D] float32 states before the first and
// after the last token (may be null: zero start, not wanted).
hipError_t wkv5_forward_launch(int64_t B, int64_t T, int64_t H, int64_t D,
                               const uint16_t* r, const uint16_t* k, const uint16_t* v,
                               const float* w, const float* u, float* o, void* ws,
                               const float* s_in, float* s_out, hipStream_t stream);

hipError_t wkv5_step_launch(int64_t B, int64_t H, float* s, const uint16_t* r,
                            const uint16_t* k, const uint16_t* v, const float* w,
                            const float* u, float* o, hipStream_t stream);

// ----- Finch (RWKV-6): per-token decay w [B, T, H, D] (step: [B, H, D]) -----
size_t wkv6_workspace_bytes(int64_t B, int64_t T, int64_t H);

hipError_t wkv6_forward_launch(int64_t B, int64_t T, int64_t H, const uint16_t* r,
                               const uint16_t* k, const uint16_t* v, const float* w,
                               const float* u, float* o, const float* s_in, float* s_out,
                               void* ws, hipStream_t stream);

hipError_t wkv6_step_launch(int64_t B, int64_t H, float* s, const uint16_t* r,
                            const uint16_t* k, const uint16_t* v, const float* w,
                            const float* u, float* o, hipStream_t stream);

}  // namespace rwkv
