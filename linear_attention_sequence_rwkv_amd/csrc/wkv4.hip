// RWKV-4 WKV kernels for gfx950: recurrent step, state init, and the
// time-parallel forward as a single-pass tiled scan.
//
// What is computed: [RWKV-digest] "RWKV - Reinventing RNNs for the
// Transformer Era" (paper digest), Method > (2) Time-mixing (WKV): WKV_t and
// its recurrent form a_t = e^{-w} a_{t-1} + e^{k_t} v_t (same for b with 1),
// WKV_t = (a_{t-1} + e^{u+k_t} v_t) / (b_{t-1} + e^{u+k_t}).  The time-parallel
// form rests on the associativity of "decay then add" (same page, atomic
// insight on the training/inference duality).
//
// Forward design (one launch, 12 bytes of HBM traffic per element plus a
// few percent of workspace):
//   * a channel block is 64*CPL channels of one sequence; each lane owns CPL
//     adjacent channels and loads them with one vector load per token;
//   * a workgroup owns one tile of one channel block: NW waves stacked along
//     time, L tokens each, k and v held in registers;
//   * each wave summarises its L tokens from an empty history; wave 0 joins
//     the NW summaries into the tile aggregate and publishes it;
//   * wave 0 then walks back over earlier tiles of the same block (decoupled
//     look-back, 16 tiles polled per round trip): aggregates are folded in
//     until an earlier tile's inclusive history ends the walk;
//   * every wave rebuilds its starting history from the tile prefix and the
//     summaries of the waves before it, rescans its tokens from registers in
//     8-token blocks with one exp2 per token (rescan_blocked) and writes y.
// A wait must only ever be on a running workgroup.  When the device holds
// every workgroup of the grid at once, tile t of a block is simply the
// (t * blocks + block)-th workgroup, whose loads go out before anything else
// (the epoch is read after them, and wave 0's first look-back poll before the
// summaries' barrier); otherwise tiles of a channel block are claimed in
// arrival order from that block's own counter (one atomic round trip before
// the loads can start, about 0.8 us of a 17 us launch).  Every
// word the kernel writes to the workspace carries the call's tag, the
// workspace epoch + 1, which the call advances once all its workgroups have
// read it; nothing is reset between calls whatever their shapes, and launches
// replayed from a captured graph stay correct.
#include "wkv4_scan.h"
#include "wkv_device.h"
#include "wkv_internal.h"

#include <mutex>


namespace rwkv {

namespace {

using namespace scan;

// Output pass of a full wave: the blocked rescan, each token's y stored as
// it is produced.
template <int L, int CPL>
__device__ __forceinline__ void emit_rows_blocked(Rsrc ry, uint32_t voff, uint32_t row_bytes,
                                                  Hist (&hs)[CPL], const float (&kk)[L][CPL],
                                                  const float (&vv)[L][CPL],
                                                  const float (&u2)[CPL],
                                                  const float (&w2)[CPL]) {
  rescan_blocked<L, CPL>(hs, kk, vv, u2, w2,
                         [&](int s, const float (&y)[CPL], const float (&)[CPL],
                             const float (&)[CPL], const float (&)[CPL]) {
                           store_row<CPL>(ry, voff, uint32_t(s) * row_bytes, y);
                         });
}

template <int L, int CPL, bool FULL>
__device__ __forceinline__ void emit_rows(Rsrc ry, uint32_t voff, uint32_t row_bytes, int n,
                                          Hist (&hs)[CPL], const float (&kk)[L][CPL],
                                          const float (&vv)[L][CPL], const float (&u2)[CPL],
                                          const float (&w2)[CPL]) {
#pragma unroll
  for (int s = 0; s < L; ++s) {
    if (FULL || s < n) {
      float ys[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) ys[c] = hist_read_push(hs[c], kk[s][c], vv[s][c], u2[c], w2[c]);
      store_row<CPL>(ry, voff, uint32_t(s) * row_bytes, ys);
    }
  }
}

// NaN over one tile's output rows: the mark of a tile that could not run.
template <int CPL, int L, int NW>
__device__ void nan_rows(int tile, int g, int wid, int T, int C, int n_cblk,
                         float* __restrict__ y) {
  constexpr int W = 64 * CPL;
  const int lane = threadIdx.x & 63;
  const int bi = g / n_cblk, cb = g - bi * n_cblk;
  const int t0 = tile * L * NW + wid * L;
  const int n = max(0, min(L, T - t0));
#pragma unroll 1
  for (int s = 0; s < n; ++s)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = cb * W + lane * CPL + c;
      if (ch < C) y[(size_t(bi) * T + t0 + s) * C + ch] = __builtin_nanf("");
    }
}

// Optional recurrent state around a forward call, in the step API's form
// (a, b, p: true sums a*e^p and b*e^p), [B, C] each; null pointers mean
// "empty history" (in) and "not wanted" (out).
struct StateIO {
  const float* a_in;
  const float* b_in;
  const float* p_in;
  float* a_out;
  float* b_out;
  float* p_out;
};

template <int CPL>
__device__ __forceinline__ void write_state(const StateIO& sio, const Hist (&h)[CPL],
                                            const float (&w2)[CPL], bool valid, size_t si) {
  if (!sio.a_out || !valid) return;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    sio.a_out[si + c] = h[c].A;
    sio.b_out[si + c] = h[c].Bd;
    sio.p_out[si + c] = hist_p(h[c], w2[c]) * kLn2;
  }
}

// Look-back of tile `tile` of channel block g (one wave, lane = channel):
// the history of every earlier tile of the block, rebuilt as
// inc(p) + agg(p+1) + ... + agg(tile-1), folded in that order for the
// nearest p (within kWin) whose inclusive history is out.  That is the order
// in which the chain of inclusive histories is built, so the result has the
// same bits whichever p the timing offers: the forward is deterministic.
// With `early`, the first poll's words (lanes < kWin: inc and agg words of
// tile-1-lane) were loaded by the caller.  A wait beyond spin_limit polls
// raises the error word and returns NaN.
template <int CPL, int TILE>
__device__ __forceinline__ void lookback(int tile, int g, int groups,
                                         const uint64_t* __restrict__ slots, uint32_t* hdr,
                                         uint32_t tag, const float (&w2)[CPL], bool early,
                                         uint64_t e_inc, uint64_t e_agg, Hist (&acc)[CPL],
                                         uint32_t spin_limit) {
  constexpr int W = 64 * CPL;
  constexpr int SLOT = 8 * W;  // words per (tile, block): agg A,B,kr,n then inc A,B,kr,n
  // Predecessor payloads loaded per round trip while folding a prefix
  // (the batch costs 8 VGPRs per payload and channel).
  constexpr int kFoldBatch = CPL == 1 ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int ch0 = lane * CPL;
  uint32_t spins = 0;
  for (;;) {
    // Poll kWin earlier tiles in one round trip: lane i reads the first
    // word of tile (tile-1-i)'s inclusive and aggregate histories.
    const int pi = tile - 1 - lane;
    bool inc_ok = false, agg_ok = false;
    if (early) {
      inc_ok = lane < kWin && pi >= 0 && tag_ok(e_inc, tag);
      agg_ok = lane < kWin && pi > 0 && tag_ok(e_agg, tag);
      early = false;
    } else if (lane < kWin && pi >= 0) {
      const uint64_t* sp = slots + (size_t(pi) * groups + g) * SLOT;
      inc_ok = tag_ok(tagged_load(sp + 4 * W), tag);
      agg_ok = pi > 0 && tag_ok(tagged_load(sp), tag);  // tile 0 has no aggregate
    }
    const uint64_t inc_mask = __ballot(inc_ok);
    const uint64_t agg_mask = __ballot(agg_ok);
    const int m = inc_mask ? int(__builtin_ctzll(inc_mask)) : kWin;
    const int a = int(__builtin_ctzll(~agg_mask));  // bits >= kWin are 0
    if (inc_mask != 0 && a >= m) {
      // Payload j = 0 is inc(tile-1-m), payload j >= 1 is agg(tile-1-m+j).
      const int p0 = tile - 1 - m;
      bool ok = true;
      for (int j0 = 0; j0 <= m && ok; j0 += kFoldBatch) {
        uint64_t x[kFoldBatch][CPL][4];
#pragma unroll
        for (int jj = 0; jj < kFoldBatch; ++jj) {
          const int j = j0 + jj;
          const uint64_t* q =
              slots + (size_t(p0 + j) * groups + g) * SLOT + (j == 0 ? 4 * W : 0) + ch0;
#pragma unroll
          for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int f = 0; f < 4; ++f)
              x[jj][c][f] = j <= m ? tagged_load(q + f * W + c) : (uint64_t(tag) << 32);
        }
#pragma unroll
        for (int jj = 0; jj < kFoldBatch; ++jj)
#pragma unroll
          for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int f = 0; f < 4; ++f) ok = ok && tag_ok(x[jj][c][f], tag);
        ok = __all(ok);  // a payload not yet visible on every lane: poll again
        if (!ok) break;
#pragma unroll
        for (int jj = 0; jj < kFoldBatch; ++jj) {
          const int j = j0 + jj;
          if (j > m) break;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const Hist h{tag_val(x[jj][c][0]), tag_val(x[jj][c][1]), tag_val(x[jj][c][2]),
                         tag_val(x[jj][c][3])};
            acc[c] = j == 0 ? h : hist_concat(acc[c], h, float(TILE), w2[c]);
          }
        }
      }
      if (ok) break;
    }
    if (++spins > spin_limit) {
      if (lane == 0) raise_error(hdr + kHdrError, kErrGaveUp);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float nan = __builtin_nanf("");
        acc[c] = Hist{nan, nan, nan, 0.f};
      }
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// EMIT = false: publish the tiles' histories only (the backward's prefix
// pass); no output rows, no state.  With `mids`, each tile also publishes the
// inclusive history at its middle (after NW/2 waves), for a consumer tiled at
// half the length.
//
// in_order != 0: the launch has checked that every workgroup of the grid can
// be resident at once, so tiles follow the launch index; the epoch advances
// when the last tile of every block has seen its prefix, which every other
// tile's published words (carrying the tag it read) have then reached, and
// that tile leaves its block's counter primed for a next call that claims.
// in_order == 0: tiles are claimed in arrival order.
//
// TAPE (with outputs): also publish the mid-tile histories in `mids`, as the
// prefix pass does, so that a backward over the same inputs can skip that
// pass (a forward for training).
//
// CB > 1: a workgroup covers CB adjacent channel blocks of one sequence
// (n_cblk % CB == 0), NW waves along time for each; wave i serves block
// i % CB at time slot i / CB.  Every block keeps its own 128-token tiles,
// histories and look-back, so the results are those of CB = 1 bit for bit;
// what changes is the memory pattern: the CB waves of a time slot read
// adjacent 256-byte pieces of the same rows together.  Tiles are claimed
// per group of CB blocks.
template <int CPL, int L, int NW, bool EMIT = true, bool TAPE = false, int CB = 1,
          int POL = kLoadStream>
__global__ __launch_bounds__(64 * NW * CB) void wkv4_fwd_tiled(
    int T, int C, int n_cblk, int groups, int n_tiles, int in_order,
    const float* __restrict__ w, const float* __restrict__ u,
    const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ y,
    uint32_t* __restrict__ hdr, uint64_t* __restrict__ counters, uint64_t* __restrict__ slots,
    StateIO sio, uint64_t* __restrict__ mids, uint32_t spin_limit) {
  constexpr int W = 64 * CPL;        // channels per block
  constexpr int TILE = L * NW;       // tokens per tile
  constexpr int SLOT = 8 * W;        // words per (tile, block): agg A,B,kr,n then inc A,B,kr,n
  __shared__ int s_tile;
  __shared__ uint32_t s_tag;
  __shared__ HistLds<W> s_sums[CB][NW];
  __shared__ HistLds<W> s_pres[CB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wid = wave / CB;         // time slot of this wave in the tile
  const int bo = wave - wid * CB;    // its block within the workgroup's CB blocks
  const int ngrp = groups / CB;      // groups of CB blocks
  const int gg = int(blockIdx.x) % ngrp;
  const int g = gg * CB + bo;
  HistLds<W>(&s_sum)[NW] = s_sums[bo];
  HistLds<W>& s_pre = s_pres[bo];
  int tile;
  if (in_order) {
    // The tile is known at once, so the loads need not wait for anything;
    // the tag is read after they are issued (below).
    tile = int(blockIdx.x) / ngrp;
  } else {
    if (threadIdx.x == 0) {
      uint32_t tg;
      s_tile = claim_tile(hdr, counters, gg, n_tiles, ngrp, tg);
      s_tag = tg;
    }
    lds_barrier();
    tile = __builtin_amdgcn_readfirstlane(s_tile);
    // Only a workspace that was never zero-filled can get here: flag it and
    // write NaN over the rows of the tile this workgroup's launch index
    // names (the caller must not mistake them for results).
    if (tile < 0 || tile >= n_tiles) {
      if (threadIdx.x == 0) raise_error(hdr + kHdrError, kErrNotZeroed);
      if (EMIT) nan_rows<CPL, L, NW>(int(blockIdx.x) / ngrp, g, wid, T, C, n_cblk, y);
      return;
    }
  }
  const int bi = g / n_cblk;
  const int cb = g - bi * n_cblk;
  const int ch0 = lane * CPL;                 // first channel of this lane in the block
  const bool valid = cb * W + ch0 < C;        // C % CPL == 0: all CPL valid or none
  const int cl = valid ? ch0 : (C - cb * W - CPL);  // loads stay in bounds
  float w2[CPL], u2[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    w2[c] = w[cb * W + cl + c] * kLog2e;
    u2[c] = u[cb * W + cl + c] * kLog2e;
  }

  const int tile_t0 = tile * TILE;
  const int t0 = tile_t0 + wid * L;
  const int n = max(0, min(L, T - t0));
  const size_t row0 = (size_t(bi) * size_t(T) + size_t(t0)) * size_t(C) + size_t(cb) * W;
  // Offsets within a wave's rows stay below 2^31 (checked by the plan).
  const uint32_t row_bytes = uint32_t(C) * 4u;
  const uint32_t span = uint32_t(L - 1) * row_bytes + uint32_t(W) * 4u;
  const Rsrc rk = make_rsrc(k + row0, span);
  const Rsrc rv = make_rsrc(v + row0, span);
  const uint32_t voff_in = uint32_t(cl) * 4u;

  float kk[L][CPL], vv[L][CPL];
  const bool full = n == L;
  if (full)
    load_rows<L, CPL, true, POL>(rk, rv, voff_in, row_bytes, n, kk, vv);
  else
    load_rows<L, CPL, false, POL>(rk, rv, voff_in, row_bytes, n, kk, vv);
  if (in_order && threadIdx.x == 0) s_tag = hdr_load(hdr, kHdrEpoch) + 1u;

  // Pass 1: this wave's tokens from an empty history, at raised issue
  // priority (the summaries gate the aggregate that later tiles wait for;
  // 8x1024x768: 16.58 -> 16.49 us over five runs).
  __builtin_amdgcn_s_setprio(2);
  if (full) {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      s_sum[wid].put(ch0 + c, summarize<L, CPL, true>(kk, vv, c, n, w2[c]));
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      s_sum[wid].put(ch0 + c, summarize<L, CPL, false>(kk, vv, c, n, w2[c]));
  }
  // Launch-order tiles: wave 0's first poll goes out before the barrier, so
  // its round trip overlaps the wait for the other waves' summaries
  // (8x1024x768: 17.4 -> 17.0 us; with claimed tiles, which arrive in a
  // stream of many generations, it measured 2% slower and is not used).
  uint64_t e_inc = 0, e_agg = 0;
  if (in_order && wid == 0 && tile > 0 && lane < kWin && tile - 1 - lane >= 0) {
    const uint64_t* sp = slots + (size_t(tile - 1 - lane) * groups + g) * SLOT;
    e_inc = tagged_load(sp + 4 * W);
    if (tile - 1 - lane > 0) e_agg = tagged_load(sp);  // tile 0 has no aggregate
  }
  lds_barrier();
  __builtin_amdgcn_s_setprio(0);
  const uint32_t tag = __builtin_amdgcn_readfirstlane(s_tag);

  // Blocks whose last tile has its prefix (in-order launches), as counted
  // before this one; read at the end so the round trip overlaps pass 2.
  uint32_t done_before = 0;
  // Tile prefix: wave 0 publishes the aggregate and looks back, at raised
  // issue priority: its short bursts of work between round trips then do not
  // queue behind other workgroups' output passes on the same SIMD
  // (8x1024x768: 16.73 -> 16.49 us).
  if (wid == 0) {
    __builtin_amdgcn_s_setprio(3);
    const int tile_n = min(TILE, T - tile_t0);
    uint64_t* mine = slots + (size_t(tile) * groups + g) * SLOT + ch0;
    Hist agg[CPL], pre[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      agg[c] = s_sum[0].get(ch0 + c);
      for (int i = 1; i < NW; ++i) {
        const int ni = max(0, min(L, T - (tile_t0 + i * L)));
        agg[c] = hist_concat(agg[c], s_sum[i].get(ch0 + c), float(ni), w2[c]);
      }
      pre[c] = hist_empty();
    }
    auto publish = [&](int kind, const Hist (&h)[CPL]) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        uint64_t* q = mine + kind * 4 * W + c;
        tagged_store(q + 0 * W, h[c].A, tag);
        tagged_store(q + 1 * W, h[c].Bd, tag);
        tagged_store(q + 2 * W, h[c].kr, tag);
        tagged_store(q + 3 * W, h[c].n, tag);
      }
    };
    if (tile == 0) {
      // History before the first token: empty, or the caller's state.
      if (sio.a_in) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const size_t si = size_t(bi) * C + size_t(cb) * W + cl + c;
          pre[c] = Hist{sio.a_in[si], sio.b_in[si], sio.p_in[si] * kLog2e, 0.f};
        }
      }
      Hist inc[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) inc[c] = hist_concat(pre[c], agg[c], float(tile_n), w2[c]);
      publish(1, inc);
      if (tile == n_tiles - 1) write_state(sio, inc, w2, valid, size_t(bi) * C + size_t(cb) * W + ch0);
    } else {
      publish(0, agg);
      Hist acc[CPL];
      lookback<CPL, TILE>(tile, g, groups, slots, hdr, tag, w2, in_order != 0, e_inc, e_agg, acc,
                          spin_limit);
      Hist inc[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        pre[c] = acc[c];
        inc[c] = hist_concat(pre[c], agg[c], float(tile_n), w2[c]);
      }
      publish(1, inc);
      if (tile == n_tiles - 1) write_state(sio, inc, w2, valid, size_t(bi) * C + size_t(cb) * W + ch0);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int c = 0; c < CPL; ++c) s_pre.put(ch0 + c, pre[c]);
    if (in_order && tile == n_tiles - 1 && lane == 0) {
      __hip_atomic_store(counters + size_t(g) * (kWkv4CounterStride / sizeof(uint64_t)),
                         uint64_t(tag + 1u) << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      done_before = hdr_add(hdr, kHdrClaimed, 1u);
    }
    if ((!EMIT || TAPE) && mids) {
      uint64_t* q = mids + (size_t(tile) * groups + g) * (4 * W) + ch0;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        Hist mid = pre[c];
        for (int i = 0; i < NW / 2; ++i) {
          const int ni = max(0, min(L, T - (tile_t0 + i * L)));
          mid = hist_concat(mid, s_sum[i].get(ch0 + c), float(ni), w2[c]);
        }
        tagged_store(q + 0 * W + c, mid.A, tag);
        tagged_store(q + 1 * W + c, mid.Bd, tag);
        tagged_store(q + 2 * W + c, mid.kr, tag);
        tagged_store(q + 3 * W + c, mid.n, tag);
      }
    }
  }
  lds_barrier();

  // Pass 2: start from the tile prefix plus the earlier waves, emit y.
  if (EMIT && n > 0) {
    Hist hs[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      hs[c] = s_pre.get(ch0 + c);
      for (int i = 0; i < wid; ++i)
        hs[c] = hist_concat(hs[c], s_sum[i].get(ch0 + c), float(L), w2[c]);
    }
    const Rsrc ry = make_rsrc(y + row0, span);
    const uint32_t voff_out = valid ? uint32_t(ch0) * 4u : kDropOffset;
    if (full)
      emit_rows_blocked<L, CPL>(ry, voff_out, row_bytes, hs, kk, vv, u2, w2);
    else
      emit_rows<L, CPL, false>(ry, voff_out, row_bytes, n, hs, kk, vv, u2, w2);
  }
  if (in_order && wid == 0 && lane == 0 && tile == n_tiles - 1 &&
      done_before == uint32_t(groups - 1)) {
    // Every block is done reading the epoch: leave the header for the next call.
    hdr_store(hdr, kHdrClaimed, 0u);
    hdr_store(hdr, kHdrEpoch, tag);
  }
}

// One thread per 4 consecutive channels of one stream: the step is
// elementwise, 36 bytes of traffic per element.  The state stays on the
// default cache policy (the next step reads it again); this token's k, v and
// the output y are touched once and go non-temporal (measured at 256 streams
// x 4096 channels: 7.0 -> 6.6 us per step).
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void step_one(float& a, float& b, float& p, float w, float u,
                                         float k, float v, float& y) {
  const float w2 = w * kLog2e;
  Hist h{a, b, p * kLog2e, 0.f};
  y = hist_read_push(h, k * kLog2e, v, u * kLog2e, w2);
  a = h.A;
  b = h.Bd;
  p = hist_p(h, w2) * kLn2;
}

__global__ __launch_bounds__(256) void wkv4_step_vec4(
    int B, int C4, float4* __restrict__ a, float4* __restrict__ b, float4* __restrict__ p,
    const float4* __restrict__ w, const float4* __restrict__ u,
    const float4* __restrict__ k, const float4* __restrict__ v, float4* __restrict__ y) {
  const int c4 = blockIdx.x * 256 + threadIdx.x;
  if (c4 >= C4) return;
  const float4 wv = w[c4], uv = u[c4];
  for (int row = blockIdx.y; row < B; row += gridDim.y) {
    const size_t i = size_t(row) * C4 + c4;
    float4 av = a[i], bv = b[i], pv = p[i];
    const f4v kx = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(k) + i);
    const f4v vx = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(v) + i);
    const float4 kv = make_float4(kx.x, kx.y, kx.z, kx.w);
    const float4 vv = make_float4(vx.x, vx.y, vx.z, vx.w);
    float4 yv;
    step_one(av.x, bv.x, pv.x, wv.x, uv.x, kv.x, vv.x, yv.x);
    step_one(av.y, bv.y, pv.y, wv.y, uv.y, kv.y, vv.y, yv.y);
    step_one(av.z, bv.z, pv.z, wv.z, uv.z, kv.z, vv.z, yv.z);
    step_one(av.w, bv.w, pv.w, wv.w, uv.w, kv.w, vv.w, yv.w);
    a[i] = av;
    b[i] = bv;
    p[i] = pv;
    __builtin_nontemporal_store(f4v{yv.x, yv.y, yv.z, yv.w}, reinterpret_cast<f4v*>(y) + i);
  }
}

__global__ __launch_bounds__(256) void wkv4_step_scalar(
    int B, int C, float* __restrict__ a, float* __restrict__ b, float* __restrict__ p,
    const float* __restrict__ w, const float* __restrict__ u,
    const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ y) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const float wc = w[c], uc = u[c];
  for (int row = blockIdx.y; row < B; row += gridDim.y) {
    const size_t i = size_t(row) * C + c;
    float av = a[i], bv = b[i], pv = p[i], yv;
    step_one(av, bv, pv, wc, uc, __builtin_nontemporal_load(k + i),
             __builtin_nontemporal_load(v + i), yv);
    a[i] = av;
    b[i] = bv;
    p[i] = pv;
    __builtin_nontemporal_store(yv, y + i);
  }
}

__global__ __launch_bounds__(256) void wkv4_state_fill(size_t n, float* __restrict__ a,
                                                       float* __restrict__ b,
                                                       float* __restrict__ p) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256) {
    a[i] = 0.f;
    b[i] = 0.f;
    p[i] = kEmptyP;
  }
}

struct Variant {
  int cpl, L, NW, cb;
  constexpr int code() const { return (cb > 1 ? cb * 100000 : 0) + cpl * 10000 + L * 100 + NW; }
};
// Instantiated tile shapes: channels per lane, tokens per wave, waves per
// block and tile, channel blocks per workgroup.
constexpr Variant kVariants[] = {{4, 8, 8, 1},  {4, 16, 4, 1}, {4, 16, 8, 1}, {2, 16, 8, 1},
                                 {2, 32, 4, 1}, {2, 16, 4, 1}, {1, 32, 8, 1}, {1, 32, 4, 1},
                                 {1, 64, 1, 1}, {1, 16, 4, 1}, {1, 32, 4, 2}, {1, 32, 4, 4}};

// Workgroups of `kern` (`block` threads, no dynamic LDS) that the current
// device holds at once, cached per device; 0 if it cannot be determined, or
// if the kTuneWkv4Order override asks for claimed tiles (tests compare the
// modes).
int64_t device_capacity(const void* kern, int block);

int64_t resident_workgroups(const void* kern, int block) {
  if (tuning(kTuneWkv4Order) == 1) return 0;
  return device_capacity(kern, block);
}

// Workgroups of `kern` that the current device holds at once (0 if unknown).
int64_t device_capacity(const void* kern, int block) {
  constexpr int kMaxDev = 64;
  struct Entry {
    const void* kern;
    int64_t n;
  };
  static std::mutex mu;
  static Entry cache[kMaxDev][32] = {};  // more than the kernels a process can launch
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (Entry& e : cache[dev]) {
    if (e.kern == kern) return e.n;
    if (e.kern == nullptr) {
      int per_cu = 0, cus = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, block, 0) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
      e.kern = kern;
      e.n = int64_t(per_cu) * cus;
      return e.n;
    }
  }
  return 0;
}

template <int CPL, int L, int NW, int CB = 1>
hipError_t launch_tiled(const Wkv4Plan& pl, int64_t T, int64_t C, const float* w,
                        const float* u, const float* k, const float* v, float* y, void* ws,
                        const StateIO& sio, hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  uint32_t* hdr = reinterpret_cast<uint32_t*>(base);
  uint64_t* counters = reinterpret_cast<uint64_t*>(base + kWkv4HeaderBytes);
  uint64_t* slots = reinterpret_cast<uint64_t*>(base + pl.slots_offset);
  const int64_t grid = pl.n_tiles * pl.groups / CB;
  const void* kern = reinterpret_cast<const void*>(&wkv4_fwd_tiled<CPL, L, NW, true, false, CB>);
  const int in_order = grid <= resident_workgroups(kern, 64 * NW * CB) ? 1 : 0;
  hipLaunchKernelGGL((wkv4_fwd_tiled<CPL, L, NW, true, false, CB>), dim3(unsigned(grid)),
                     dim3(64 * NW * CB), 0, stream, int(T), int(C), int(pl.n_cblk), int(pl.groups),
                     int(pl.n_tiles), in_order, w, u, k, v, y, hdr, counters, slots, sio, nullptr,
                     wkv4_spin_limit());
  return hipGetLastError();
}

// Tiles (128 tokens x 64 channels) from which the plan groups channel
// blocks: far more than the ~1000 such workgroups the device holds at once.
constexpr int64_t kGroupedMinTiles = 8192;

}  // namespace

bool wkv4_plan_fixed(int64_t B, int64_t T, int64_t C, int cpl, int L, int NW, Wkv4Plan* plan) {
  Wkv4Plan p;
  p.cb = 1;
  p.cpl = cpl;
  p.L = L;
  p.NW = NW;
  p.tile = int64_t(L) * NW;
  p.n_tiles = (T + p.tile - 1) / p.tile;
  p.n_cblk = (C + 64 * cpl - 1) / (64 * cpl);
  p.groups = B * p.n_cblk;
  // Tiles, token and channel indices are 32-bit in the kernel; byte offsets
  // within a wave's rows are 32-bit, below the 2^31 drop offset.
  if (p.n_tiles * p.groups >= (int64_t(1) << 31) || T > kWkv4MaxT ||
      p.groups >= (int64_t(1) << 31) ||
      (int64_t(L - 1) * C + 64 * cpl) * 4 >= (int64_t(1) << 31))
    return false;
  const size_t ctr_bytes = size_t(p.groups) * kWkv4CounterStride;
  p.slots_offset = (kWkv4HeaderBytes + ctr_bytes + 255) / 256 * 256;
  p.ws_bytes = p.slots_offset + size_t(p.n_tiles) * size_t(p.groups) * 8 * 64 * size_t(cpl) *
                                    sizeof(uint64_t);
  *plan = p;
  return true;
}

int wkv4_grouped_cb(int64_t B, int64_t T, int64_t C) {
  // Grids far beyond what the device holds at once (B=1 T=65536 C=5120:
  // 40,960 tiles) group two adjacent channel blocks per workgroup: the rows
  // then come in 512-byte pieces, which HBM serves faster (B=1 T=65536
  // C=5120: 748 -> 718 us; a copy through the same pattern 703 -> 674 us).
  // Grids the device holds at once run faster with one block per workgroup
  // (8x1024x768: 16.1 against 17.4 us).
  const int64_t n_cblk = (C + 63) / 64;
  return n_cblk % 2 == 0 && B * n_cblk * ((T + 127) / 128) >= kGroupedMinTiles ? 2 : 1;
}

bool wkv4_plan(int64_t B, int64_t T, int64_t C, Wkv4Plan* plan) {
  // One channel per lane, 32 tokens per wave, 4 waves per tile: about 116
  // VGPRs (4 waves per SIMD).  Measured faster than wider vector loads with
  // several channels per lane, which lengthen each lane's serial scan.
  int cpl = 1, L = 32, NW = 4, cb = 1;
  if (T <= 64) {
    L = 64;
    NW = 1;
  }
  if (L == 32) cb = wkv4_grouped_cb(B, T, C);
  // An override applies where its channel width divides C and its channel
  // blocks per workgroup divide the blocks of a sequence.
  if (const int code = tuning(kTuneWkv4Tile)) {
    for (const Variant& vv : kVariants)
      if (vv.code() == code && C % vv.cpl == 0 &&
          ((C + 64 * vv.cpl - 1) / (64 * vv.cpl)) % vv.cb == 0) {
        cpl = vv.cpl;
        L = vv.L;
        NW = vv.NW;
        cb = vv.cb;
      }
  }
  if (!wkv4_plan_fixed(B, T, C, cpl, L, NW, plan)) return false;
  plan->cb = cb;
  return true;
}

bool wkv4_keep_rows(const Wkv4Plan& pl, int64_t T, int64_t C) {
  const int64_t B = pl.groups / pl.n_cblk;
  return 8 * B * T * C <= kKeepRowBytes;
}

uint32_t wkv4_spin_limit() {
  const int s = tuning(kTuneWkv4Spin);
  return s > 0 ? uint32_t(s) : kSpinLimit;
}

bool wkv4_variant_exists(int code) {
  for (const Variant& vv : kVariants)
    if (vv.code() == code) return true;
  return false;
}

namespace {

// The prefix pass (EMIT = false) or the training forward (TAPE = true) of
// the backward's plan: 1 channel per lane, 32 tokens x 4 waves, CB channel
// blocks per workgroup.
template <bool EMIT, bool TAPE, int CB, int POL>
hipError_t launch_prefix_like(const Wkv4Plan& pl, int64_t T, int64_t C, const float* w,
                              const float* u, const float* k, const float* v, float* y,
                              void* ws, void* mids, hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  uint32_t* hdr = reinterpret_cast<uint32_t*>(base);
  uint64_t* counters = reinterpret_cast<uint64_t*>(base + kWkv4HeaderBytes);
  uint64_t* slots = reinterpret_cast<uint64_t*>(base + pl.slots_offset);
  const int64_t grid = pl.n_tiles * pl.groups / CB;
  const StateIO none{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  const void* kern =
      reinterpret_cast<const void*>(&wkv4_fwd_tiled<1, 32, 4, EMIT, TAPE, CB, POL>);
  const int in_order = grid <= resident_workgroups(kern, 256 * CB) ? 1 : 0;
  hipLaunchKernelGGL((wkv4_fwd_tiled<1, 32, 4, EMIT, TAPE, CB, POL>), dim3(unsigned(grid)),
                     dim3(256 * CB), 0, stream, int(T), int(C), int(pl.n_cblk), int(pl.groups),
                     int(pl.n_tiles), in_order, w, u, k, v, y, hdr, counters, slots, none,
                     static_cast<uint64_t*>(mids), wkv4_spin_limit());
  return hipGetLastError();
}

}  // namespace

hipError_t wkv4_prefix_launch(const Wkv4Plan& pl, int64_t T, int64_t C, const float* w,
                              const float* u, const float* k, const float* v, void* ws,
                              void* mids, hipStream_t stream) {
  if (pl.cpl != 1 || pl.L != 32 || pl.NW != 4) return hipErrorInvalidValue;
  const bool keep = wkv4_keep_rows(pl, T, C);
  if (pl.cb == 2)
    return keep ? launch_prefix_like<false, false, 2, kLoadKeep>(pl, T, C, w, u, k, v, nullptr,
                                                                ws, mids, stream)
                : launch_prefix_like<false, false, 2, kLoadStream>(pl, T, C, w, u, k, v, nullptr,
                                                                  ws, mids, stream);
  if (pl.cb == 1)
    return keep ? launch_prefix_like<false, false, 1, kLoadKeep>(pl, T, C, w, u, k, v, nullptr,
                                                                ws, mids, stream)
                : launch_prefix_like<false, false, 1, kLoadStream>(pl, T, C, w, u, k, v, nullptr,
                                                                  ws, mids, stream);
  return hipErrorInvalidValue;
}

hipError_t wkv4_forward_tape_launch(const Wkv4Plan& pl, int64_t T, int64_t C, const float* w,
                                   const float* u, const float* k, const float* v, float* y,
                                   void* ws, void* mids, hipStream_t stream) {
  if (pl.cpl != 1 || pl.L != 32 || pl.NW != 4) return hipErrorInvalidValue;
  // The backward that follows reads k and v again: where they fit the
  // memory-side cache, load them with the default policy so they stay there.
  const bool keep = wkv4_keep_rows(pl, T, C);
  if (pl.cb == 2)
    return keep ? launch_prefix_like<true, true, 2, kLoadKeep>(pl, T, C, w, u, k, v, y, ws,
                                                              mids, stream)
                : launch_prefix_like<true, true, 2, kLoadStream>(pl, T, C, w, u, k, v, y, ws,
                                                                mids, stream);
  if (pl.cb == 1)
    return keep ? launch_prefix_like<true, true, 1, kLoadKeep>(pl, T, C, w, u, k, v, y, ws,
                                                              mids, stream)
                : launch_prefix_like<true, true, 1, kLoadStream>(pl, T, C, w, u, k, v, y, ws,
                                                                mids, stream);
  return hipErrorInvalidValue;
}

hipError_t wkv4_forward_launch(const Wkv4Plan& pl, int64_t B, int64_t T, int64_t C,
                               const float* w, const float* u, const float* k,
                               const float* v, float* y, void* ws, const float* a_in,
                               const float* b_in, const float* p_in, float* a_out,
                               float* b_out, float* p_out, hipStream_t stream) {
  (void)B;
  const StateIO sio{a_in, b_in, p_in, a_out, b_out, p_out};
  switch ((pl.cb > 1 ? pl.cb * 100000 : 0) + pl.cpl * 10000 + pl.L * 100 + pl.NW) {
    case 213204: return launch_tiled<1, 32, 4, 2>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 413204: return launch_tiled<1, 32, 4, 4>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 40808: return launch_tiled<4, 8, 8>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 41604: return launch_tiled<4, 16, 4>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 41608: return launch_tiled<4, 16, 8>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 21608: return launch_tiled<2, 16, 8>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 23204: return launch_tiled<2, 32, 4>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 21604: return launch_tiled<2, 16, 4>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 13208: return launch_tiled<1, 32, 8>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 13204: return launch_tiled<1, 32, 4>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 16401: return launch_tiled<1, 64, 1>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    case 11604: return launch_tiled<1, 16, 4>(pl, T, C, w, u, k, v, y, ws, sio, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t wkv4_state_init_launch(int64_t B, int64_t C, float* a, float* b, float* p,
                                  hipStream_t stream) {
  const size_t n = size_t(B) * size_t(C);
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(wkv4_state_fill, dim3(unsigned(blocks)), dim3(256), 0, stream, n, a, b, p);
  return hipGetLastError();
}

hipError_t wkv4_step_launch(int64_t B, int64_t C, float* a, float* b, float* p,
                            const float* w, const float* u, const float* k, const float* v,
                            float* y, hipStream_t stream) {
  const unsigned rows = unsigned(B < 65535 ? B : 65535);
  if (C % 4 == 0) {
    const int64_t C4 = C / 4;
    const dim3 grid(unsigned((C4 + 255) / 256), rows);
    hipLaunchKernelGGL(wkv4_step_vec4, grid, dim3(256), 0, stream, int(B), int(C4),
                       reinterpret_cast<float4*>(a), reinterpret_cast<float4*>(b),
                       reinterpret_cast<float4*>(p), reinterpret_cast<const float4*>(w),
                       reinterpret_cast<const float4*>(u), reinterpret_cast<const float4*>(k),
                       reinterpret_cast<const float4*>(v), reinterpret_cast<float4*>(y));
  } else {
    const dim3 grid(unsigned((C + 255) / 256), rows);
    hipLaunchKernelGGL(wkv4_step_scalar, grid, dim3(256), 0, stream, int(B), int(C), a, b, p,
                       w, u, k, v, y);
  }
  return hipGetLastError();
}

}  // namespace rwkv
