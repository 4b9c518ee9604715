// RWKV-4 WKV backward for gfx950: the gradients of L = sum gy * WKV with
// respect to w, u, k and v.
//
// What is differentiated: [RWKV-digest] "RWKV - Reinventing RNNs for the
// Transformer Era" (paper digest), Method > (2) Time-mixing (WKV): WKV_t is
// a weighted mean of v_i, i <= t, with log-weights k_i - (t-1-i) w (i < t)
// and u + k_t (i = t).  The pages give no derivatives.  With D_t the sum of
// the weights and p_{t,i} = weight / D_t, dWKV_t/dv_i = p_{t,i} and
// dWKV_t/d(log-weight_{t,i}) = p_{t,i} (v_i - WKV_t), so
//   gv_i = sum_{t>=i} g_t p_{t,i},
//   gk_i = sum_{t>=i} g_t p_{t,i} (v_i - WKV_t),
//   gu   = sum_t g_t p_{t,t} (v_t - WKV_t),
//   gw   = -sum_t sum_{i<t} (t-1-i) g_t p_{t,i} (v_i - WKV_t).
// For i < t, p_{t,i} = 2^{k2_i} 2^{-(t-1-i) w2} / D_t (base-2 domain), so
// the sums over t > i are reverse-time histories of the values g_t / D_t and
// g_t WKV_t / D_t, plus their age-weighted versions for gw.  D_t is carried
// as 2^{sc_t} den_t (den_t in [1, t+1]): the values g_t / den_t with "keys"
// -sc_t.
//
// Three launches on one stream:
//   1. the forward's tiled scan without its output pass (128-token tiles)
//      publishes every tile's inclusive forward history in the workspace,
//      and the one after each tile's first 64 tokens;
//   2. wkv4_bwd_tiled (64-token tiles): tiles are claimed from the last one
//      backwards; each wave rescans its tokens forward from the published
//      prefix to recover WKV_t, D_t and p_{t,t} in registers, summarises
//      its reverse history, and wave 0 publishes the tile's reverse aggregate
//      and folds the later tiles' (deterministic look-back, as in the
//      forward); every wave then runs the reverse scan, writing gk and gv and
//      summing its lanes' gw and gu terms, which go to a per-(tile, sequence)
//      slot;
//   3. wkv4_bwd_reduce sums those slots per channel in a fixed order.
// Every result is deterministic: no float atomics, folds in chain order.
#include "wkv4_scan.h"
#include "wkv_device.h"
#include "wkv_internal.h"

namespace rwkv {

namespace {

using namespace scan;

// Sums over later tokens t of c_t 2^{-sc_t - (t-1-i) w2} for c_t = g_t / den_t
// (G) and g_t WKV_t / den_t (H), and the same weighted by the age t-1-i (G1,
// H1), seen from a position i.  The common scale is anchored as in Hist:
// kr - n w2, kr the key (-sc) of the anchor term and n the decays since.
struct RevHist {
  float G, H, G1, H1, kr, n;
};

__device__ __forceinline__ RevHist rev_empty() { return RevHist{0.f, 0.f, 0.f, 0.f, kEmptyP, 0.f}; }

// y: the ny tokens right after position i, seen from i; x: the tokens after
// those, seen from i + ny.  Returns all of them seen from i: x's ages grow by
// ny (its moments gain ny times its plain sums) and it decays by ny steps.
__device__ __forceinline__ RevHist rev_concat(const RevHist& y, const RevHist& x, float ny,
                                              float w2) {
  const float xg1 = fmaf(ny, x.G, x.G1);
  const float xh1 = fmaf(ny, x.H, x.H1);
  const float nx = x.n + ny;
  const float d = fmaf(-(nx - y.n), w2, x.kr - y.kr);  // scale of x minus scale of y
  const float e = exp2_fast(-fabsf(d));
  const bool keep = d >= 0.f;
  RevHist r;
  r.G = keep ? fmaf(e, y.G, x.G) : fmaf(e, x.G, y.G);
  r.H = keep ? fmaf(e, y.H, x.H) : fmaf(e, x.H, y.H);
  r.G1 = keep ? fmaf(e, y.G1, xg1) : fmaf(e, xg1, y.G1);
  r.H1 = keep ? fmaf(e, y.H1, xh1) : fmaf(e, xh1, y.H1);
  r.kr = keep ? x.kr : y.kr;
  r.n = keep ? nx : y.n;
  return r;
}

template <int W>
struct RevLds {
  float f[6][W];
  __device__ __forceinline__ RevHist get(int ch) const {
    return RevHist{f[0][ch], f[1][ch], f[2][ch], f[3][ch], f[4][ch], f[5][ch]};
  }
  __device__ __forceinline__ void put(int ch, const RevHist& h) {
    f[0][ch] = h.G;
    f[1][ch] = h.H;
    f[2][ch] = h.G1;
    f[3][ch] = h.H1;
    f[4][ch] = h.kr;
    f[5][ch] = h.n;
  }
};

constexpr int kRevFields = 6;

// One channel per lane, L tokens per wave, NW waves per tile.
template <int L, int NW, int POL>
__global__ __launch_bounds__(64 * NW) void wkv4_bwd_tiled(
    int T, int C, int n_cblk, int groups, int n_tiles,
    const float* __restrict__ w, const float* __restrict__ u,
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ gy,
    float* __restrict__ gk, float* __restrict__ gv,
    const uint64_t* __restrict__ fwd_slots,  // inclusive forward histories (launch 1)
    const uint64_t* __restrict__ fwd_mids,   // and those after the first half of its tiles
    uint32_t* __restrict__ hdr, uint64_t* __restrict__ counters, uint64_t* __restrict__ slots,
    uint64_t* __restrict__ part_w, uint64_t* __restrict__ part_u, uint32_t spin_limit) {
  constexpr int W = 64;
  constexpr int TILE = L * NW;
  constexpr int FSLOT = 8 * W;             // forward slot: agg A,B,kr,n then inc A,B,kr,n
  constexpr int RSLOT = 2 * kRevFields * W;  // reverse slot: agg fields then inc fields
  __shared__ int s_tile;
  __shared__ uint32_t s_tag;
  __shared__ HistLds<W> s_fsum[NW];
  __shared__ RevLds<W> s_rsum[NW];
  __shared__ RevLds<W> s_rsuf;
  __shared__ float s_red[2][NW][W];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = int(blockIdx.x) % groups;
  if (threadIdx.x == 0) {
    uint32_t tg;
    const int t = claim_tile(hdr, counters, g, n_tiles, groups, tg);
    s_tile = t < 0 ? -1 : n_tiles - 1 - t;  // the last tile first
    s_tag = tg;
  }
  __syncthreads();
  const int tile = __builtin_amdgcn_readfirstlane(s_tile);
  const uint32_t tag = __builtin_amdgcn_readfirstlane(s_tag);
  if (tile < 0 || tile >= n_tiles) {
    // A workspace that was never zero-filled: flag it, and write NaN over the
    // gradient rows of the tile this workgroup's launch index names.
    if (threadIdx.x == 0) raise_error(hdr + kHdrError, kErrNotZeroed);
    const int lt = n_tiles - 1 - int(blockIdx.x) / groups;
    const int bi = g / n_cblk, cb = g - bi * n_cblk;
    const int ch = cb * 64 + (threadIdx.x & 63);
    const int t0 = lt * L * NW + int(threadIdx.x >> 6) * L;
    const int n = max(0, min(L, T - t0));
    if (ch < C) {
#pragma unroll 1
      for (int s = 0; s < n; ++s) {
        const size_t i = (size_t(bi) * T + t0 + s) * C + ch;
        gk[i] = __builtin_nanf("");
        gv[i] = __builtin_nanf("");
      }
      // and the tile's gw, gu slots, so that the sums over tiles are NaN too
      if (threadIdx.x < 64) {
        const size_t pi = (size_t(lt) * (groups / n_cblk) + bi) * size_t(C) + size_t(ch);
        tagged_store(part_w + pi, __builtin_nanf(""), tag);
        tagged_store(part_u + pi, __builtin_nanf(""), tag);
      }
    }
    return;
  }
  const int bi = g / n_cblk;
  const int cb = g - bi * n_cblk;
  const int ch = lane;
  const bool valid = cb * W + ch < C;
  const int cl = valid ? ch : (C - cb * W - 1);  // loads stay in bounds
  const float w2 = w[cb * W + cl] * kLog2e;
  const float u2 = u[cb * W + cl] * kLog2e;

  const int tile_t0 = tile * TILE;
  const int t0 = tile_t0 + wid * L;
  const int n = max(0, min(L, T - t0));
  const size_t row0 = (size_t(bi) * size_t(T) + size_t(t0)) * size_t(C) + size_t(cb) * W;
  const uint32_t row_bytes = uint32_t(C) * 4u;
  const uint32_t span = uint32_t(L - 1) * row_bytes + uint32_t(W) * 4u;
  const Rsrc rk = make_rsrc(k + row0, span);
  const Rsrc rv = make_rsrc(v + row0, span);
  const Rsrc rg = make_rsrc(gy + row0, span);
  const uint32_t voff_in = uint32_t(cl) * 4u;

  float kk[L][1], vv[L][1], gg[L];
  const bool full = n == L;
  if (full)
    load_rows<L, 1, true, POL>(rk, rv, voff_in, row_bytes, n, kk, vv);
  else
    load_rows<L, 1, false, POL>(rk, rv, voff_in, row_bytes, n, kk, vv);
#pragma unroll
  for (int s = 0; s < L; ++s) {
    float t1[1] = {0.f};
    if (full || s < n) load_row<1, POL>(rg, voff_in, uint32_t(s) * row_bytes, t1);
    gg[s] = t1[0];
  }

  // Forward: this wave's summary, then its prefix = published inclusive
  // history of the previous tile + the summaries of the earlier waves.
  s_fsum[wid].put(ch, full ? summarize<L, 1, true>(kk, vv, 0, n, w2)
                           : summarize<L, 1, false>(kk, vv, 0, n, w2));
  __syncthreads();
  float yy[L], ll[L], pp[L];
  {
    Hist h = hist_empty();
    if (tile > 0) {
      // the prefix pass's tiles are twice as long: the history after this
      // tile's predecessor p is the inclusive history of prefix tile p / 2
      // (p odd) or the one after its first half (p even)
      const int pk = tile - 1;
      const uint64_t* q =
          (pk & 1) ? fwd_slots + (size_t(pk >> 1) * groups + g) * FSLOT + 4 * W + ch
                   : fwd_mids + (size_t(pk >> 1) * groups + g) * (4 * W) + ch;
      h = Hist{tag_val(q[0]), tag_val(q[W]), tag_val(q[2 * W]), tag_val(q[3 * W])};
    }
    for (int i = 0; i < wid; ++i) h = hist_concat(h, s_fsum[i].get(ch), float(L), w2);
    if (full) {
      Hist hs[1] = {h};
      const float u2a[1] = {u2}, w2a[1] = {w2};
      rescan_blocked<L, 1>(hs, kk, vv, u2a, w2a,
                           [&](int s, const float (&y)[1], const float (&sc)[1],
                               const float (&pe)[1], const float (&rd)[1]) {
                             yy[s] = y[0];
                             ll[s] = sc[0];
                             pp[s] = pe[0];
                             gg[s] *= rd[0];  // g_t / den_t from here on
                           });
    } else {
#pragma unroll
      for (int s = 0; s < L; ++s) {
        yy[s] = 0.f;
        ll[s] = 0.f;
        pp[s] = 0.f;
        if (s < n) {
          float rd;
          yy[s] = read_push_ld(h, kk[s][0], vv[s][0], u2, w2, ll[s], pp[s], rd);
          gg[s] *= rd;  // g_t / den_t from here on
        }
      }
    }
  }

  // Reverse summary of this wave's tokens seen from position t0 - 1: token
  // t0 + s has age s, key -sc and value g / den.  Fixed reference: the
  // largest exponent, so every factor is at most 1.
  {
    float P = kEmptyP;
#pragma unroll
    for (int s = 0; s < L; ++s)
      if (full || s < n) P = fmaxf(P, fmaf(-float(s), w2, -ll[s]));
    RevHist r = rev_empty();
    if (n > 0) {
      r.kr = P;
#pragma unroll
      for (int s = 0; s < L; ++s) {
        if (full || s < n) {
          const float e = exp2_fast(fmaf(-float(s), w2, -ll[s]) - P);
          const float eg = e * gg[s];
          const float egy = eg * yy[s];
          r.G += eg;
          r.H += egy;
          r.G1 = fmaf(float(s), eg, r.G1);
          r.H1 = fmaf(float(s), egy, r.H1);
        }
      }
    }
    s_rsum[wid].put(ch, r);
  }
  __syncthreads();

  // Tile suffix: wave 0 publishes the tile's reverse aggregate and folds the
  // later tiles in chain order (deterministic, as in the forward).
  if (wid == 0) {
    const int tile_n = min(TILE, T - tile_t0);
    RevHist agg = s_rsum[NW - 1].get(ch);
    for (int i = NW - 2; i >= 0; --i) agg = rev_concat(s_rsum[i].get(ch), agg, float(L), w2);
    uint64_t* mine = slots + (size_t(tile) * groups + g) * RSLOT + ch;
    auto publish = [&](int kind, const RevHist& h) {
      uint64_t* q = mine + kind * kRevFields * W;
      tagged_store(q + 0 * W, h.G, tag);
      tagged_store(q + 1 * W, h.H, tag);
      tagged_store(q + 2 * W, h.G1, tag);
      tagged_store(q + 3 * W, h.H1, tag);
      tagged_store(q + 4 * W, h.kr, tag);
      tagged_store(q + 5 * W, h.n, tag);
    };
    RevHist suf = rev_empty();  // later tiles, seen from this tile's last token
    if (tile == n_tiles - 1) {
      publish(1, agg);
    } else {
      publish(0, agg);
      uint32_t spins = 0;
      for (;;) {
        // lane i polls tile tile+1+i
        const int pi = tile + 1 + lane;
        bool inc_ok = false, agg_ok = false;
        if (lane < kWin && pi < n_tiles) {
          const uint64_t* sp = slots + (size_t(pi) * groups + g) * RSLOT;
          inc_ok = tag_ok(tagged_load(sp + kRevFields * W), tag);
          agg_ok = pi < n_tiles - 1 && tag_ok(tagged_load(sp), tag);  // the last has no aggregate
        }
        const uint64_t inc_mask = __ballot(inc_ok);
        const uint64_t agg_mask = __ballot(agg_ok);
        const int m = inc_mask ? int(__builtin_ctzll(inc_mask)) : kWin;
        const int a = int(__builtin_ctzll(~agg_mask));
        if (inc_mask != 0 && a >= m) {
          // suffix = agg(tile+1) + (... + (agg(tile+m) + inc(tile+1+m)))
          bool ok = true;
          RevHist acc = rev_empty();
          for (int j = m; j >= 0 && ok; --j) {
            const uint64_t* q = slots + (size_t(tile + 1 + j) * groups + g) * RSLOT +
                                (j == m ? kRevFields * W : 0) + ch;
            uint64_t x[kRevFields];
#pragma unroll
            for (int f = 0; f < kRevFields; ++f) x[f] = tagged_load(q + f * W);
#pragma unroll
            for (int f = 0; f < kRevFields; ++f) ok = ok && tag_ok(x[f], tag);
            ok = __all(ok);
            if (!ok) break;
            const RevHist hj{tag_val(x[0]), tag_val(x[1]), tag_val(x[2]),
                             tag_val(x[3]), tag_val(x[4]), tag_val(x[5])};
            acc = j == m ? hj : rev_concat(hj, acc, float(TILE), w2);
          }
          if (ok) {
            suf = acc;
            break;
          }
        }
        if (++spins > spin_limit) {
          if (lane == 0) raise_error(hdr + kHdrError, kErrGaveUp);
          const float nan = __builtin_nanf("");
          suf = RevHist{nan, nan, nan, nan, nan, 0.f};
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      publish(1, rev_concat(agg, suf, float(tile_n), w2));
    }
    s_rsuf.put(ch, suf);
  }
  __syncthreads();

  // Reverse scan of this wave from its last token, starting from the later
  // waves of the tile and the tile suffix.
  float acc_w = 0.f, acc_u = 0.f;
  if (n > 0) {
    RevHist h = s_rsuf.get(ch);
    for (int i = NW - 1; i > wid; --i) h = rev_concat(s_rsum[i].get(ch), h, float(L), w2);
    const Rsrc rgk = make_rsrc(gk + row0, span);
    const Rsrc rgv = make_rsrc(gv + row0, span);
    const uint32_t voff_out = valid ? uint32_t(ch) * 4u : kDropOffset;
#pragma unroll
    for (int s = L - 1; s >= 0; --s) {
      if (full || s < n) {
        const float k2 = kk[s][0], vi = vv[s][0], g_ = gg[s], yi = yy[s];
        const float ek = exp2_fast(fmaf(-h.n, w2, h.kr + k2));  // 2^{k2} x the scale
        const float own = g_ * pp[s];
        const float dvy = vi - yi;
        float o_v[1] = {fmaf(ek, h.G, own)};
        float o_k[1] = {fmaf(own, dvy, ek * fmaf(vi, h.G, -h.H))};
        acc_w = fmaf(ek, fmaf(vi, h.G1, -h.H1), acc_w);
        acc_u = fmaf(own, dvy, acc_u);
        store_row<1>(rgv, voff_out, uint32_t(s) * row_bytes, o_v);
        store_row<1>(rgk, voff_out, uint32_t(s) * row_bytes, o_k);
        // move the view to the token before: ages grow by one, then this
        // token's own term (key -sc, value g / den, age 0) joins
        h.G1 += h.G;
        h.H1 += h.H;
        const float d = fmaf(-(h.n + 1.f), w2, h.kr + ll[s]);
        const float e = exp2_fast(-fabsf(d));
        const bool keep = d >= 0.f;
        const float gyv = g_ * yi;
        h.G = keep ? fmaf(e, g_, h.G) : fmaf(e, h.G, g_);
        h.H = keep ? fmaf(e, gyv, h.H) : fmaf(e, h.H, gyv);
        h.G1 = keep ? h.G1 : e * h.G1;
        h.H1 = keep ? h.H1 : e * h.H1;
        h.kr = keep ? h.kr : -ll[s];
        h.n = keep ? h.n + 1.f : 0.f;
      }
    }
  }
  s_red[0][wid][ch] = acc_w;
  s_red[1][wid][ch] = acc_u;
  __syncthreads();
  if (wid == 0 && valid) {
    float sw = 0.f, su = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      sw += s_red[0][i][ch];
      su += s_red[1][i][ch];
    }
    const size_t pi = (size_t(tile) * (groups / n_cblk) + bi) * size_t(C) + size_t(cb) * W + ch;
    tagged_store(part_w + pi, sw, tag);
    tagged_store(part_u + pi, su, tag);
  }
}

// gw[c] = -(sum of the gw slots of channel c), gu[c] = sum of its gu slots.
// A workgroup takes 64
// channels (lane = channel, so every load is one coalesced row) and its 16
// waves take every 16th row, four rows in flight per wave; the 16 wave sums
// are added in a fixed order.  Double precision throughout.
constexpr int kRedWaves = 16;

__global__ __launch_bounds__(64 * kRedWaves) void wkv4_bwd_reduce(
    int C, int rows, const uint64_t* __restrict__ part_w, const uint64_t* __restrict__ part_u,
    float* __restrict__ gw, float* __restrict__ gu) {
  __shared__ double s_w[kRedWaves][64], s_u[kRedWaves][64];
  const int cl = threadIdx.x & 63;
  const int r0 = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + cl;
  double sw = 0.0, su = 0.0;
  if (c < C) {
    int r = r0;
    for (; r + 3 * kRedWaves < rows; r += 4 * kRedWaves) {
      float xw[4], xu[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xw[j] = tag_val(part_w[size_t(r + j * kRedWaves) * C + c]);
        xu[j] = tag_val(part_u[size_t(r + j * kRedWaves) * C + c]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sw += double(xw[j]);
        su += double(xu[j]);
      }
    }
    for (; r < rows; r += kRedWaves) {
      sw += double(tag_val(part_w[size_t(r) * C + c]));
      su += double(tag_val(part_u[size_t(r) * C + c]));
    }
  }
  s_w[r0][cl] = sw;
  s_u[r0][cl] = su;
  __syncthreads();
  if (r0 == 0 && c < C) {
    double tw = 0.0, tu = 0.0;
#pragma unroll
    for (int g = 0; g < kRedWaves; ++g) {
      tw += s_w[g][cl];
      tu += s_u[g][cl];
    }
    gw[c] = float(-tw);
    gu[c] = float(tu);
  }
}

// Reverse-pass tiles: 64 tokens, 16 on each of 4 waves (8 on each of 8
// waves measured slower: 59.5 against 56.2 us at B=8 T=1024 C=768); the
// prefix pass runs the forward's 128-token tiles (32 tokens x 4 waves).
constexpr int kBwdL = 16;
constexpr int kBwdNW = 4;

}  // namespace

bool wkv4_backward_plan(int64_t B, int64_t T, int64_t C, Wkv4BwdPlan* plan) {
  Wkv4BwdPlan p;
  // The prefix pass streams k, v in the forward's 128-token tiles; the
  // reverse pass holds six values per token and lane, so its tiles are half
  // that long and read the prefix pass's mid-tile histories too.
  if (!wkv4_plan_fixed(B, T, C, 1, 32, 4, &p.fwd)) return false;
  // Two channel blocks per workgroup on grids far beyond the device's
  // capacity, as the forward (the prefix pass and the training forward share
  // it; the reverse pass claims through every block's counter, raising any
  // the prefix pass left to its own tag first).
  p.fwd.cb = wkv4_grouped_cb(B, T, C);
  const int64_t groups = p.fwd.groups;
  p.rev_tiles = (T + kBwdL * kBwdNW - 1) / (kBwdL * kBwdNW);
  if (p.rev_tiles * groups >= (int64_t(1) << 31)) return false;
  // Both passes share the header and counters at the start (the prefix pass
  // leaves each counter primed with the reverse pass's tag); everything after
  // them holds tagged words only, so the layout of any later call of another
  // shape finds nothing but smaller tags wherever its counters land.
  p.mid_offset = (p.fwd.ws_bytes + 255) / 256 * 256;
  const size_t mid_bytes = size_t(p.fwd.n_tiles) * size_t(groups) * 4 * 64 * sizeof(uint64_t);
  p.rev_slots_offset = (p.mid_offset + mid_bytes + 255) / 256 * 256;
  const size_t rev_slot_bytes =
      size_t(p.rev_tiles) * size_t(groups) * 2 * kRevFields * 64 * sizeof(uint64_t);
  p.part_offset = (p.rev_slots_offset + rev_slot_bytes + 255) / 256 * 256;
  p.part_rows = p.rev_tiles * B;
  const size_t part_bytes = size_t(p.part_rows) * size_t(C) * sizeof(uint64_t);
  p.ws_bytes = p.part_offset + 2 * ((part_bytes + 255) / 256 * 256);
  *plan = p;
  return true;
}

hipError_t wkv4_backward_launch(const Wkv4BwdPlan& pl, int64_t B, int64_t T, int64_t C,
                                const float* w, const float* u, const float* k,
                                const float* v, const float* gy, float* gw, float* gu,
                                float* gk, float* gv, void* ws, bool prefix_ready,
                                hipStream_t stream) {
  (void)B;
  char* base = static_cast<char*>(ws);
  uint64_t* mids = reinterpret_cast<uint64_t*>(base + pl.mid_offset);
  // 1. forward prefixes of every tile and half tile, unless a forward for
  //    training left them
  hipError_t e = hipSuccess;
  if (!prefix_ready) {
    e = wkv4_prefix_launch(pl.fwd, T, C, w, u, k, v, base, mids, stream);
    if (e != hipSuccess) return e;
  }
  // 2. reverse scan, on the same header and counters
  const uint64_t* fwd_slots = reinterpret_cast<const uint64_t*>(base + pl.fwd.slots_offset);
  uint32_t* hdr = reinterpret_cast<uint32_t*>(base);
  uint64_t* counters = reinterpret_cast<uint64_t*>(base + kWkv4HeaderBytes);
  uint64_t* slots = reinterpret_cast<uint64_t*>(base + pl.rev_slots_offset);
  uint64_t* part_w = reinterpret_cast<uint64_t*>(base + pl.part_offset);
  const size_t part_bytes = size_t(pl.part_rows) * size_t(C) * sizeof(uint64_t);
  uint64_t* part_u =
      reinterpret_cast<uint64_t*>(base + pl.part_offset + (part_bytes + 255) / 256 * 256);
  const unsigned grid = unsigned(pl.rev_tiles * pl.fwd.groups);
  if (wkv4_keep_rows(pl.fwd, T, C))
    hipLaunchKernelGGL((wkv4_bwd_tiled<kBwdL, kBwdNW, kLoadKeep>), dim3(grid), dim3(64 * kBwdNW),
                       0, stream, int(T), int(C), int(pl.fwd.n_cblk), int(pl.fwd.groups),
                       int(pl.rev_tiles), w, u, k, v, gy, gk, gv, fwd_slots, mids, hdr, counters,
                       slots, part_w, part_u, wkv4_spin_limit());
  else
    hipLaunchKernelGGL((wkv4_bwd_tiled<kBwdL, kBwdNW, kLoadStream>), dim3(grid),
                       dim3(64 * kBwdNW), 0, stream, int(T), int(C), int(pl.fwd.n_cblk),
                       int(pl.fwd.groups), int(pl.rev_tiles), w, u, k, v, gy, gk, gv, fwd_slots,
                       mids, hdr, counters, slots, part_w, part_u, wkv4_spin_limit());
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 3. gw, gu
  hipLaunchKernelGGL(wkv4_bwd_reduce, dim3(unsigned((C + 63) / 64)), dim3(64 * kRedWaves), 0,
                     stream, int(C),
                     int(pl.part_rows), part_w, part_u, gw, gu);
  return hipGetLastError();
}

hipError_t wkv4_forward_train_launch(const Wkv4BwdPlan& pl, int64_t T, int64_t C,
                                     const float* w, const float* u, const float* k,
                                     const float* v, float* y, void* ws, hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  return wkv4_forward_tape_launch(pl.fwd, T, C, w, u, k, v, y, base, base + pl.mid_offset,
                                  stream);
}

}  // namespace rwkv
