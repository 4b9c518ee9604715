/*
 * rwkv_wkv.h - C ABI of the RWKV WKV operator library for AMD MI355X (gfx950).
 *
 * Sources, by page title and section (the formulas each call evaluates):
 *   [RWKV-digest]  "RWKV - Reinventing RNNs for the Transformer Era" (Korean
 *                  paper digest, irregular6612.github.io), Method > core
 *                  components > (2) Time-mixing (WKV): the WKV_t equation and
 *                  its recurrent form with states a_t, b_t.
 *   [RWKV-summary] "RWKV: Reinventing RNNs for the Transformer Era"
 *                  (flashpapers.ai summary), sec. 3 "The WKV Operator".
 *   [Eagle-Finch]  "RWKV-5 Eagle and RWKV-6 Finch" (ql.gl blog), sections
 *                  "Eagle: extending vector memory to matrix memory" and
 *                  "Finch: making the recurrence respond to the input".
 *
 * Common rules for every entry point:
 *   - Pointers named as device pointers are device memory of the current HIP
 *     device, owned by the caller, dense row-major with the last index
 *     fastest, and 16-byte aligned.  The library never allocates, frees,
 *     synchronises or prints.
 *   - Calls enqueue work on `stream` (0 = the null stream) and return without
 *     waiting.  A fault inside a kernel surfaces at the caller's next
 *     synchronisation, not in the return value.
 *   - Arguments are checked on the host before any HIP call.  A failed check
 *     returns a negative status and enqueues nothing.  Zero-sized problems
 *     return RWKV_OK and enqueue nothing.
 *   - Values are not checked: NaN/Inf in the inputs propagate to the outputs.
 *   - Outputs must not overlap inputs, except the in-place recurrent state.
 *   - All entry points are thread-safe; concurrent calls that share a
 *     workspace or a state buffer race and are not allowed.
 */
#ifndef RWKV_WKV_H
#define RWKV_WKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle (the same typedef as in hip_runtime_api.h). */
typedef struct ihipStream_t* hipStream_t;

#define RWKV_WKV_ABI_VERSION 1

/* Status codes returned by every int-valued entry point. */
#define RWKV_OK               0
#define RWKV_ERR_NULLPTR     -1  /* a required pointer is NULL */
#define RWKV_ERR_SHAPE       -2  /* negative size, or a size product overflows */
#define RWKV_ERR_UNSUPPORTED -3  /* a shape this build does not implement */
#define RWKV_ERR_WORKSPACE   -4  /* workspace NULL or smaller than required */
#define RWKV_ERR_ALIGN       -5  /* a pointer is not 16-byte aligned */
#define RWKV_ERR_HIP         -6  /* a HIP launch failed; see rwkv_last_hip_error */

/* Version of this ABI (RWKV_WKV_ABI_VERSION of the build). */
int rwkv_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* rwkv_status_str(int status);

/* hipError_t value of the last RWKV_ERR_HIP returned on this thread (0 if none). */
int rwkv_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Plan overrides, for tests and tuning sweeps; results stay within the same
 * accuracy bounds whatever the setting, except under RWKV_TUNE_WKV4_SPIN,
 * which exists to make look-backs give up.  Each key holds 0 (the built-in
 * plan) or an override.  The values start from the environment, read once at the
 * first call that plans anything (RWKV_WKV4_TILE="cpl,L,NW",
 * RWKV_WKV4_ORDER=claim, RWKV_WKV5_DV, RWKV_WKV5_SEGS, RWKV_WKV6_DV,
 * RWKV_WKV6_SEGS), and rwkv_set_tuning changes them for the whole process.
 * They change the plan and therefore the workspace sizes: query a workspace
 * size under the setting it will be used with (a call whose workspace is too
 * small for the current setting returns RWKV_ERR_WORKSPACE).  Changing a
 * setting while another thread plans a call races with that call's plan.
 * rwkv_set_tuning returns RWKV_ERR_UNSUPPORTED for an unknown key or value.
 * ---------------------------------------------------------------------- */
#define RWKV_TUNE_WKV4_TILE  1  /* [cb*100000 +] cpl*10000 + L*100 + NW of a compiled RWKV-4
                                   forward shape (cb: channel blocks per workgroup, 1 if absent):
                                   40808 41604 41608 21608 23204 21604 13208 13204 16401 11604
                                   213204 413204 */
#define RWKV_TUNE_WKV4_ORDER 2  /* 1: RWKV-4 tiles claimed in arrival order even where the
                                   whole grid is resident (same results, bit for bit) */
#define RWKV_TUNE_WKV5_DV    3  /* value columns per Eagle workgroup: 16, 32 or 64 */
#define RWKV_TUNE_WKV5_SEGS  4  /* Eagle time segments, 1..4096 (each >= 4 chunks) */
#define RWKV_TUNE_WKV6_DV    5  /* value columns per Finch workgroup: 32 or 64 */
#define RWKV_TUNE_WKV6_SEGS  6  /* Finch time segments, 1..4096 (each >= 4 chunks) */
#define RWKV_TUNE_WKV4_SPIN  7  /* polls an RWKV-4 look-back (forward or backward) makes
                                   before it gives up, sets error bit 0 and writes NaN;
                                   0: the default, 2^24.  For tests of that path: a small
                                   limit makes tiles give up that would have succeeded. */
int rwkv_set_tuning(int key, int value);
int rwkv_get_tuning(int key);

/* ------------------------------------------------------------------------
 * Device-side errors of the RWKV-4 scans.  The first 32-bit word of a
 * forward or backward workspace is an error word, 0 while all is well:
 *   bit 0 (1): a tile waited for its predecessors longer than its spin limit
 *              (about 2^24 polls) and gave up; its outputs are NaN;
 *   bit 1 (2): a tile claim found a workspace that was never zero-filled;
 *              the rows of that tile are NaN.
 * The backward's gw and gu, summed over every tile, are NaN in the channels
 * of a tile of the call that gave up or could not be claimed.
 * Either bit means the outputs of the calls made since the word was last 0
 * are not to be trusted.  The word is sticky: zero-filling the workspace
 * (always allowed between calls) clears it.
 * rwkv_wkv4_workspace_error enqueues on `stream` a copy of the word into
 * *err (device memory or pinned host memory; valid once the stream has
 * reached that point).  It checks only its own arguments.
 * ---------------------------------------------------------------------- */
int rwkv_wkv4_workspace_error(const void* ws, size_t ws_bytes, uint32_t* err,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * RWKV-4 time-parallel forward.   [RWKV-digest] (2) Time-mixing, WKV_t;
 * [RWKV-summary] sec. 3 "The WKV Operator".
 *
 * For every batch b, token t and channel c (0-based):
 *   y[b,t,c] = ( sum_{i<t} e^{-(t-1-i) w[c] + k[b,i,c]} v[b,i,c] + e^{u[c]+k[b,t,c]} v[b,t,c] )
 *            / ( sum_{i<t} e^{-(t-1-i) w[c] + k[b,i,c]}          + e^{u[c]+k[b,t,c]} )
 * i.e. the history starts empty at t = 0.
 *
 *   w  [C]      float32  decay rate >= 0; one step back multiplies by e^{-w}
 *   u  [C]      float32  current-token bonus
 *   k, v [B,T,C] float32
 *   y  [B,T,C]  float32  output
 *   ws, ws_bytes         device workspace of at least
 *                        rwkv_wkv4_forward_workspace(B,T,C) bytes.  It must be
 *                        zero-filled before its first use; each call leaves it
 *                        ready for the next call on the same stream.  Its words
 *                        are tagged with a 32-bit count of the launches made on
 *                        it (one per call here, two for a backward), so it must
 *                        be zero-filled again at least once every 2^30 calls,
 *                        graph replays included.  A call whose workspace size
 *                        is 0 accepts ws == NULL.
 * Accuracy: max |y - exact| <= 1e-4 * S, where S is the same weighted mean
 * taken over |v| (float32 arithmetic, hardware exp2 and reciprocal).
 * Limit: T <= 2^24 - 64 per call (decay counts are held in float32, exact
 * for integers up to 2^24); longer sequences are cut and chained through
 * rwkv_wkv4_forward_state.  Larger T returns RWKV_ERR_UNSUPPORTED (and the
 * workspace query 0).  The same limit holds for the backward and training
 * calls.
 * ---------------------------------------------------------------------- */
size_t rwkv_wkv4_forward_workspace(int64_t B, int64_t T, int64_t C);
int rwkv_wkv4_forward(int64_t B, int64_t T, int64_t C,
                      const float* w, const float* u,
                      const float* k, const float* v,
                      float* y,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * RWKV-4 forward that allocates nothing and takes no workspace.  For callers
 * that cannot allocate or hand over device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * Arguments, results (bit for bit) and accuracy as rwkv_wkv4_forward.  The
 * look-back workspace is a 32 MiB device array inside the library, one per
 * GPU, held until the process ends: shapes whose
 * rwkv_wkv4_forward_workspace(B, T, C) exceeds 32 MiB (under the current
 * plan overrides) return RWKV_ERR_WORKSPACE and enqueue nothing.  The array
 * is zero-filled by a kernel on `stream` at the first call on each device
 * (and again every 2^30 calls); it keeps the last call's contents, which the
 * next call needs no clearing of.  Make the first call on each device
 * outside graph capture (it also looks up the array's device address); a
 * fill recorded into a graph is repeated at the next call made outside one.
 * Launches replayed from a captured graph are not counted: past 2^32
 * launches without a fill the 32-bit call tags wrap, after which a call of
 * a shape other than the last one's may find its tiles unclaimable and write
 * NaN over its rows.  Every call on one GPU shares the array:
 * calls that overlap in time on that GPU (other streams, other threads)
 * race and are not allowed.  The array's error word is not exposed; a tile
 * that cannot run still writes NaN over its rows, as in rwkv_wkv4_forward.
 * ---------------------------------------------------------------------- */
int rwkv_wkv4_forward_noalloc(int64_t B, int64_t T, int64_t C,
                              const float* w, const float* u,
                              const float* k, const float* v,
                              float* y, hipStream_t stream);

/* ------------------------------------------------------------------------
 * RWKV-4 backward: gradients of L = sum_{b,t,c} gy[b,t,c] * y[b,t,c], with y
 * the output of rwkv_wkv4_forward (empty starting history).
 * [RWKV-digest] (2) Time-mixing, WKV_t; the pages give no derivatives.  With
 * p[t,i] the normalised weight of token i in y[t] (per b, c):
 *   gv[b,i,c] = sum_{t>=i} gy[b,t,c] p[t,i]
 *   gk[b,i,c] = sum_{t>=i} gy[b,t,c] p[t,i] (v[b,i,c] - y[b,t,c])
 *   gu[c]     = sum_{b,t} gy[b,t,c] p[t,t] (v[b,t,c] - y[b,t,c])
 *   gw[c]     = -sum_{b,t} sum_{i<t} (t-1-i) gy[b,t,c] p[t,i] (v[b,i,c] - y[b,t,c])
 *
 *   w, u        [C]      float32  as for the forward
 *   k, v, gy    [B,T,C]  float32
 *   gw, gu      [C]      float32  output (overwritten, summed over b and t)
 *   gk, gv      [B,T,C]  float32  output
 *   ws, ws_bytes         device workspace of at least
 *                        rwkv_wkv4_backward_workspace(B,T,C) bytes, zero-filled
 *                        before its first use and again at least once every
 *                        2^30 calls (as for the forward; it is not
 *                        interchangeable with a forward workspace).
 * Deterministic: repeated calls give the same bits.  Accuracy: each gradient
 * within 1e-4 of the same sum taken over absolute terms (|gy|, and
 * |v| + |y| for v - y).
 * ---------------------------------------------------------------------- */
size_t rwkv_wkv4_backward_workspace(int64_t B, int64_t T, int64_t C);
int rwkv_wkv4_backward(int64_t B, int64_t T, int64_t C,
                       const float* w, const float* u,
                       const float* k, const float* v, const float* gy,
                       float* gw, float* gu, float* gk, float* gv,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * RWKV-4 forward and backward for training, sharing one workspace.
 * [RWKV-digest] (2) Time-mixing, WKV_t: the forward's time-parallel scan
 * computes every tile's history before the tile; the backward needs exactly
 * those histories.  rwkv_wkv4_forward_train computes y as rwkv_wkv4_forward
 * does (same accuracy bound; the tile shape is the backward's, so the bits
 * can differ from rwkv_wkv4_forward's) and leaves the histories in `ws`;
 * rwkv_wkv4_backward_after_forward then returns what rwkv_wkv4_backward
 * returns, bit for bit, without recomputing them (one read of k and v less).
 *
 *   arguments   as for rwkv_wkv4_forward / rwkv_wkv4_backward
 *   ws, ws_bytes         a BACKWARD workspace: at least
 *                        rwkv_wkv4_backward_workspace(B,T,C) bytes, zero-filled
 *                        before its first use and again at least once every
 *                        2^30 calls.
 * The backward call must follow the forward call on the same stream, with the
 * same B, T, C, w, u, k, v and workspace, and no other call on that workspace
 * in between; otherwise its results are undefined (nothing checks this).
 * ---------------------------------------------------------------------- */
int rwkv_wkv4_forward_train(int64_t B, int64_t T, int64_t C,
                            const float* w, const float* u,
                            const float* k, const float* v,
                            float* y,
                            void* ws, size_t ws_bytes, hipStream_t stream);
int rwkv_wkv4_backward_after_forward(int64_t B, int64_t T, int64_t C,
                                     const float* w, const float* u,
                                     const float* k, const float* v, const float* gy,
                                     float* gw, float* gu, float* gk, float* gv,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * RWKV-4 recurrent state.   [RWKV-digest] (2) Time-mixing, recurrent form
 *   a_t = e^{-w} a_{t-1} + e^{k_t} v_t,   b_t = e^{-w} b_{t-1} + e^{k_t}.
 * The library stores the sums scaled: a_true = a * e^{p}, b_true = b * e^{p},
 * three float32 arrays a, b, p of shape [B,C].  Only a/b and log(b)+p are
 * meaningful; the triple itself is not unique.
 *
 * rwkv_wkv4_state_init: empty history (a = b = 0, p = -1e38).
 * ---------------------------------------------------------------------- */
int rwkv_wkv4_state_init(int64_t B, int64_t C, float* a, float* b, float* p,
                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * RWKV-4 forward continuing from, and handing on, a recurrent state.
 * [RWKV-digest] (2) Time-mixing: the recurrent form carries the whole
 * history in (a, b), so a sequence may be cut anywhere and resumed.
 *
 * As rwkv_wkv4_forward, except that the history before token 0 is the state
 * (a_in, b_in, p_in) instead of empty, and the state after token T-1 is
 * written to (a_out, b_out, p_out), in the representation described for
 * rwkv_wkv4_state_init below.  Each triple is given whole or left NULL
 * (RWKV_ERR_NULLPTR if only part of one is given): a NULL input triple means
 * the empty history, a NULL output triple means the state is not wanted.
 * The output triple may be the input triple (update in place); otherwise the
 * state arrays must not overlap each other or k, v, y.  With both NULL this
 * is rwkv_wkv4_forward.  The same workspace rules and accuracy apply, the
 * scale S then including the state's terms.
 * ---------------------------------------------------------------------- */
int rwkv_wkv4_forward_state(int64_t B, int64_t T, int64_t C,
                            const float* w, const float* u,
                            const float* k, const float* v,
                            float* y,
                            const float* a_in, const float* b_in, const float* p_in,
                            float* a_out, float* b_out, float* p_out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * RWKV-4 fused single-token step.   [RWKV-digest] (2) Time-mixing:
 *   y = (a_{t-1} + e^{u+k} v) / (b_{t-1} + e^{u+k})   using the OLD state,
 * then the state advances in place with this token's k, v.
 *
 *   a, b, p  [B,C]  float32  state, read and updated in place
 *   w, u     [C]    float32  as for the forward
 *   k, v     [B,C]  float32  this token
 *   y        [B,C]  float32  output
 * N steps from rwkv_wkv4_state_init give the same y as the forward over the
 * same N tokens (within the forward's accuracy bound).
 * ---------------------------------------------------------------------- */
int rwkv_wkv4_step(int64_t B, int64_t C,
                   float* a, float* b, float* p,
                   const float* w, const float* u,
                   const float* k, const float* v,
                   float* y, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Eagle (RWKV-5) matrix-state forward.   [Eagle-Finch] "Eagle":
 *   s' = diag(w) s + k^T v,   wkv' = s + diag(u) k^T v,  read by r.
 * Per batch b and head h, with a D x D state s[i][j] (key i, value j) that
 * starts at zero:
 *   o[b,t,h,j] = sum_i r[b,t,h,i] * ( s_t[i][j] + u[h,i] k[b,t,h,i] v[b,t,h,j] )
 *   s_{t+1}[i][j] = w[h,i] s_t[i][j] + k[b,t,h,i] v[b,t,h,j]
 *
 *   r, k, v  [B,T,H,D]  bfloat16 bit patterns (uint16)
 *   w        [H,D]      float32 decay factor in [0, 1] (the section's
 *                       exp(-exp(omega)) lies in (0, 1)); factors below
 *                       2^-126 act as 2^-126.  A head with some w outside
 *                       [0, 1], or NaN, is still computed, by the exact
 *                       float32 recurrence (serially over T: slow).
 *   u        [H,D]      float32 current-token bonus
 *   o        [B,T,H,D]  float32 output
 *   D must be 64 and H < 65536 (RWKV_ERR_UNSUPPORTED otherwise).
 *   ws, ws_bytes: at least rwkv_wkv5_forward_workspace(B,T,H,D) bytes (may
 *   be 0, then ws may be NULL); no zero-fill needed.
 * Accuracy: max |o - exact| <= 2e-2 * o_abs, where o_abs is the same sum
 * over |r|, |k|, |v|, |u| (bf16 products, float32 accumulation).
 * ---------------------------------------------------------------------- */
size_t rwkv_wkv5_forward_workspace(int64_t B, int64_t T, int64_t H, int64_t D);
int rwkv_wkv5_forward(int64_t B, int64_t T, int64_t H, int64_t D,
                      const uint16_t* r, const uint16_t* k, const uint16_t* v,
                      const float* w, const float* u,
                      float* o,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Eagle forward continuing from, and handing on, a matrix state.
 * [Eagle-Finch] "Eagle": the state s carries the whole history.
 *
 * As rwkv_wkv5_forward, except that s starts at s_in instead of zero, and
 * the state after the last token (s_T) is written to s_out.
 *   s_in, s_out  [B,H,D,D]  float32, s[b,h,i,j] = s[i][j] of (b, h); either
 *                           may be NULL (start at zero / not wanted).  s_out
 *                           may equal s_in (update in place); otherwise it
 *                           must not overlap any other argument.
 * With T = 0 nothing is enqueued (s_out is not written).  Accuracy as for
 * rwkv_wkv5_forward with |s_in| included in o_abs; s_out meets the same
 * bound against the state of that magnitude recurrence.
 * ---------------------------------------------------------------------- */
int rwkv_wkv5_forward_state(int64_t B, int64_t T, int64_t H, int64_t D,
                            const uint16_t* r, const uint16_t* k, const uint16_t* v,
                            const float* w, const float* u,
                            float* o,
                            const float* s_in, float* s_out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Eagle single-token step.   [Eagle-Finch] "Eagle": one application of
 *   o = r (s + diag(u) k^T v),   s <- diag(w) s + k^T v.
 *
 *   s        [B,H,D,D]  float32 state, read and updated in place
 *   r, k, v  [B,H,D]    bfloat16 bit patterns of this token
 *   w, u     [H,D]      float32 as for the forward
 *   o        [B,H,D]    float32 output
 *   D must be 64.  Exact float32 arithmetic on the bf16 inputs; T steps
 *   from a zero state match rwkv_wkv5_forward over the same T tokens within
 *   the forward's bound.
 * ---------------------------------------------------------------------- */
int rwkv_wkv5_step(int64_t B, int64_t H, int64_t D,
                   float* s,
                   const uint16_t* r, const uint16_t* k, const uint16_t* v,
                   const float* w, const float* u,
                   float* o, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Finch (RWKV-6) forward: the Eagle recurrence with a decay per token.
 * [Eagle-Finch] "Finch": the decay becomes data-dependent.  Read as the Eagle
 * update with token t's own decay, applied to the state before its k^T v:
 *   o[b,t,h,j] = sum_i r[b,t,h,i] * ( s_t[i][j] + u[h,i] k[b,t,h,i] v[b,t,h,j] )
 *   s_{t+1}[i][j] = w[b,t,h,i] s_t[i][j] + k[b,t,h,i] v[b,t,h,j]
 *
 *   r, k, v  [B,T,H,D]  bfloat16 bit patterns (uint16)
 *   w        [B,T,H,D]  float32 decay factor of each token, in (0, 1]
 *                       (factors below 2^-126 act as 2^-126)
 *   u        [H,D]      float32 current-token bonus
 *   o        [B,T,H,D]  float32 output
 *   s_in, s_out [B,H,D,D] float32 states before the first / after the last
 *                       token, either may be NULL (zero start / not wanted);
 *                       s_out may equal s_in.
 *   ws, ws_bytes: at least rwkv_wkv6_forward_workspace(B,T,H,D) bytes (may be
 *   0, then ws may be NULL); no zero-fill needed.
 *   D must be 64 and H < 65536 (RWKV_ERR_UNSUPPORTED otherwise).
 * Accuracy: as rwkv_wkv5_forward, against the same magnitude recurrence with
 * the per-token decays.
 * ---------------------------------------------------------------------- */
size_t rwkv_wkv6_forward_workspace(int64_t B, int64_t T, int64_t H, int64_t D);
int rwkv_wkv6_forward(int64_t B, int64_t T, int64_t H, int64_t D,
                      const uint16_t* r, const uint16_t* k, const uint16_t* v,
                      const float* w, const float* u,
                      float* o,
                      const float* s_in, float* s_out,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Finch single-token step: as rwkv_wkv5_step with this token's decay.
 *   s        [B,H,D,D]  float32 state, read and updated in place
 *   r, k, v  [B,H,D]    bfloat16 bit patterns of this token
 *   w        [B,H,D]    float32 this token's decay factors
 *   u        [H,D]      float32
 *   o        [B,H,D]    float32 output
 * ---------------------------------------------------------------------- */
int rwkv_wkv6_step(int64_t B, int64_t H, int64_t D,
                   float* s,
                   const uint16_t* r, const uint16_t* k, const uint16_t* v,
                   const float* w, const float* u,
                   float* o, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RWKV_WKV_H */
