"""fp64 CPU oracle for the RWKV WKV operators.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library and imports
nothing but NumPy.

Every function is the plain, slow, obviously correct form of what the pages
define, evaluated in float64 on the exact values handed to the GPU (float32
or bf16 inputs upcast to float64).  Sources, by page title and section:

* [RWKV-digest] "RWKV - Reinventing RNNs for the Transformer Era" (Korean
  paper digest, irregular6612.github.io), section Method > core components >
  (2) Time-mixing (WKV): the WKV_t equation and its recurrent form with the
  states a_t, b_t.
* [RWKV-summary] "RWKV: Reinventing RNNs for the Transformer Era"
  (flashpapers.ai summary), section 3 "How It Works" > "The WKV Operator".
* [Eagle-Finch] "RWKV-5 Eagle and RWKV-6 Finch" (ql.gl blog), section
  "Eagle: extending vector memory to matrix memory": the update
  s' = diag(w) s + k^T v, the read-out wkv' = s + diag(u) k^T v, and the
  decay parameterisation w = exp(-exp(omega)); section "Finch: making the
  recurrence respond to the input": the decay becomes data-dependent, i.e.
  a w_t per token (and channel) in the same update.

Conventions (readings of the pages where they are silent or garbled):

* RWKV-4 ``w`` is the positive decay *rate*; one step back multiplies by
  exp(-w).  The token immediately before t carries no decay, the one two
  back carries exp(-w) (0-based: weight exp(-(t-1-i) w + k_i) for i < t).
* RWKV-4 ``u`` is a per-channel bonus for the current token.
* The history starts empty (no terms), as the sums start at the first token.
* Eagle ``k^T v`` is an outer product indexed [key i][value j]; ``diag(w)``
  scales key rows; the receptance contracts the key index; the output reads
  the state *before* the current token's update.
* Finch: token t's decay w_t [key i] multiplies the state before token t's
  k^T v is added, s_{t+1} = diag(w_t) s_t + k_t^T v_t (the Eagle update with
  w replaced by w_t); u stays per (head, key channel).

RWKV-4 backward: the pages give WKV_t but not its derivatives.  They are
obtained here by differentiating the definition (chain rule through the
log-weights), and pinned by central finite differences of ``wkv4_direct``,
by float64 autograd of an independent torch transcription of the
definition, and by the k-shift and v-offset invariants.

Pins (tests/test_oracle.py): the direct O(T^2) sum against the recurrence,
closed forms (T=1, constant v, k=0 geometric series with the simulator's
w=0.5/u=1 defaults, w=0 prefix softmax against scipy, very large w), the
k-shift / v-affine / convex-hull invariants, Eagle recurrence against its
unrolled sum, Eagle w=1 against a masked matrix product, Eagle D=1 against
scipy.signal.lfilter, and linearity; Finch recurrence against its unrolled
sum, Finch with a constant decay against Eagle, Finch with no decay on one
channel as a prefix sum, a hand-worked case fixing when a token's decay
applies, split sequences and the scale bound.  Planted mistakes (a dropped
bonus term, the sign of w flipped, the decay one step early, a transposed
Eagle state, the decay on the value index, Finch's decay applied after the
add) each fail at least one pin.  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "wkv4_direct", "wkv4_recurrent", "wkv4_scale", "wkv4_empty_state",
    "wkv4_step", "wkv4_canonical_state",
    "wkv4_backward_direct", "wkv4_backward_recurrent", "wkv4_backward_scale",
    "wkv5_recurrent", "wkv5_unrolled", "wkv5_scale", "wkv5_step",
    "wkv6_step", "wkv6_recurrent", "wkv6_unrolled", "wkv6_scale",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# RWKV-4
# ---------------------------------------------------------------------------

def wkv4_direct(w, u, k, v):
    """WKV_t written out as the pages define it (O(T^2); tiny inputs only).

    [RWKV-digest] (2) Time-mixing, WKV_t equation; [RWKV-summary] sec. 3,
    "The WKV Operator".  For each (b, t, c) the output is the weighted mean
    of v_0..v_t with log-weights -(t-1-i) w + k_i for the past tokens i < t
    and u + k_t for the current token.  The largest log-weight is subtracted
    before exponentiating (this leaves the ratio unchanged).

    w, u: [C]; k, v: [B, T, C].  Returns y [B, T, C] float64.
    """
    w, u, k, v = _f64(w), _f64(u), _f64(k), _f64(v)
    B, T, C = k.shape
    y = np.empty((B, T, C))
    for t in range(T):
        back = (t - 1 - np.arange(t, dtype=np.float64))  # decay steps per past token
        logw_past = k[:, :t, :] - back[None, :, None] * w[None, None, :]
        logw_now = (u[None, :] + k[:, t, :])[:, None, :]
        logw = np.concatenate([logw_past, logw_now], axis=1)  # [B, t+1, C]
        vals = v[:, : t + 1, :]
        top = logw.max(axis=1, keepdims=True)
        wt = np.exp(logw - top)
        y[:, t, :] = (wt * vals).sum(axis=1) / wt.sum(axis=1)
    return y


def wkv4_empty_state(B, C):
    """Empty history: numerator and denominator sums with no terms.

    The state is (num, den, ref): the true sums are num*exp(ref) and
    den*exp(ref).  ref=-inf with num=den=0 encodes "no terms yet".
    """
    return (np.zeros((B, C)), np.zeros((B, C)), np.full((B, C), -np.inf))


def wkv4_step(state, w, u, k_t, v_t):
    """One token of the recurrent form.  Returns (y_t, new_state).

    [RWKV-digest] (2) Time-mixing, recurrent form:
      WKV_t = (a_{t-1} + e^{u+k_t} v_t) / (b_{t-1} + e^{u+k_t}),
      a_t = e^{-w} a_{t-1} + e^{k_t} v_t,   b_t = e^{-w} b_{t-1} + e^{k_t}.
    The output uses the state *before* token t; then the state advances.
    a, b are carried as (num, den) times exp(ref) so that exp never
    overflows; this scaling is not on the pages and does not change a/b.
    """
    num, den, ref = state
    w, u, k_t, v_t = _f64(w), _f64(u), _f64(k_t), _f64(v_t)
    with np.errstate(invalid="ignore", over="ignore"):
        # output: history (scaled by exp(ref)) plus the bonus term exp(u + k_t)
        cur = u + k_t
        top = np.maximum(ref, cur)
        f_hist = np.exp(ref - top)
        f_cur = np.exp(cur - top)
        y = (num * f_hist + v_t * f_cur) / (den * f_hist + f_cur)
        # advance: decay the history by exp(-w), add exp(k_t) * (v_t, 1)
        dec = ref - w
        top2 = np.maximum(dec, k_t)
        g_hist = np.exp(dec - top2)
        g_new = np.exp(k_t - top2)
        num2 = num * g_hist + v_t * g_new
        den2 = den * g_hist + g_new
    return y, (num2, den2, top2)


def wkv4_recurrent(w, u, k, v, state=None):
    """Whole-sequence output via the recurrent form, any length.

    w, u: [C]; k, v: [B, T, C].  ``state`` (optional) is the history before
    the first token in this module's (num, den, ref) form; default empty.
    Returns (y [B, T, C] float64, final state).
    """
    k, v = _f64(k), _f64(v)
    B, T, C = k.shape
    st = wkv4_empty_state(B, C) if state is None else state
    y = np.empty((B, T, C))
    for t in range(T):
        y[:, t, :], st = wkv4_step(st, w, u, k[:, t, :], v[:, t, :])
    return y, st


def wkv4_scale(w, u, k, v):
    """Condition scale S_t = sum_i alpha_i |v_i| / sum_i alpha_i.

    The same weighted mean as WKV_t, taken over |v|.  S_t >= |WKV_t|; it is
    the natural magnitude against which a rounding error in a convex
    combination is measured.
    """
    y, _ = wkv4_recurrent(w, u, k, np.abs(_f64(v)))
    return y


def wkv4_canonical_state(state):
    """Representation-free view of a state: (mean, log of the denominator).

    mean = num/den and log(den) + ref do not depend on how the sums are
    scaled, so any two correct state triples agree on them.
    """
    num, den, ref = state
    with np.errstate(divide="ignore", invalid="ignore"):
        return num / den, np.log(den) + ref


# ---------------------------------------------------------------------------
# RWKV-4 backward: gradients of L = sum_{b,t,c} gy[b,t,c] * WKV[b,t,c]
# ---------------------------------------------------------------------------
#
# With alpha_{t,i} the weight of token i in WKV_t (exp(k_i - (t-1-i) w) for
# i < t, exp(u + k_t) for i = t), D_t = sum_i alpha_{t,i} and
# p_{t,i} = alpha_{t,i} / D_t, WKV_t = sum_i p_{t,i} v_i, hence
#   d WKV_t / d v_i            = p_{t,i},
#   d WKV_t / d log alpha_{t,i} = p_{t,i} (v_i - WKV_t),
# and log alpha_{t,i} is k_i - (t-1-i) w (i < t) or u + k_t (i = t).


def wkv4_backward_direct(w, u, k, v, gy):
    """The four gradients by the definition above, O(T^2) (tiny inputs).

    w, u: [C]; k, v, gy: [B, T, C].  Returns (gw [C], gu [C], gk [B, T, C],
    gv [B, T, C]); gw and gu are summed over batch and time.
    """
    w, u = _f64(w), _f64(u)
    k, v, gy = _f64(k), _f64(v), _f64(gy)
    B, T, C = k.shape
    gk, gv = np.zeros((B, T, C)), np.zeros((B, T, C))
    gw, gu = np.zeros(C), np.zeros(C)
    for t in range(T):
        age = (t - 1 - np.arange(t))[None, :, None].astype(np.float64)   # [1, t, 1]
        logit = np.concatenate([k[:, :t] - age * w, (u + k[:, t])[:, None]], axis=1)
        a = np.exp(logit - logit.max(axis=1, keepdims=True))
        p = a / a.sum(axis=1, keepdims=True)                               # [B, t+1, C]
        y = (p * v[:, :t + 1]).sum(axis=1)                                 # [B, C]
        g = gy[:, t][:, None]                                              # [B, 1, C]
        gv[:, :t + 1] += g * p
        dlog = g * p * (v[:, :t + 1] - y[:, None])                         # d L / d log alpha
        gk[:, :t + 1] += dlog
        gu += dlog[:, t].sum(axis=0)
        gw -= (dlog[:, :t] * age).sum(axis=(0, 1))
    return gw, gu, gk, gv


def _wkv4_backward(w, u, k, v, gy, absolute):
    """Reverse-time evaluation shared by the gradients and their magnitudes.

    Forward: WKV_t and log D_t from the recurrent form.  Reverse, for the
    terms t > i of each sum:
      G_i  = sum_{t>i} gy_t e^{-(t-1-i) w - log D_t},      H_i  likewise with gy_t WKV_t,
      G'_i = sum_{t>i} (t-1-i) gy_t e^{-(t-1-i) w - log D_t}, H'_i likewise,
    so that G_{i-1} = e^{-w} G_i + gy_i / D_i and G'_{i-1} = e^{-w} (G'_i + G_i).
    Then (p_ii = e^{u + k_i} / D_i)
      gv_i = gy_i p_ii + e^{k_i} G_i
      gk_i = gy_i p_ii (v_i - WKV_i) + e^{k_i} (v_i G_i - H_i)
      gu   = sum_i gy_i p_ii (v_i - WKV_i)
      gw   = -sum_i e^{k_i} (v_i G'_i - H'_i).
    With ``absolute`` every term is replaced by a bound on its magnitude
    (|gy| for gy, |v_i| + |WKV_t| for v_i - WKV_t).  Exponentials are taken
    relative to a per-(b, c) shift, the smallest log D_t, so every stored
    factor is at most 1.
    """
    w, u = _f64(w), _f64(u)
    k, v, gy = _f64(k), _f64(v), _f64(gy)
    B, T, C = k.shape
    y = np.empty((B, T, C))
    logd = np.empty((B, T, C))
    st = wkv4_empty_state(B, C)
    with np.errstate(divide="ignore", invalid="ignore"):
        for t in range(T):
            num, den, ref = st
            logd[:, t] = np.logaddexp(np.log(den) + ref, u + k[:, t])
            y[:, t], st = wkv4_step(st, w, u, k[:, t], v[:, t])
    if absolute:
        gy = np.abs(gy)
    shift = logd.min(axis=1)                              # [B, C]
    decay = np.exp(-w)
    G, H, G1, H1 = (np.zeros((B, C)) for _ in range(4))
    gk, gv = np.empty((B, T, C)), np.empty((B, T, C))
    gw, gu = np.zeros((B, C)), np.zeros((B, C))
    for i in range(T - 1, -1, -1):
        p_ii = np.exp(u + k[:, i] - logd[:, i])
        ek = np.exp(k[:, i] - shift)
        g, vi, yi = gy[:, i], v[:, i], y[:, i]
        if absolute:
            d_own = np.abs(vi) + np.abs(yi)
            gv[:, i] = g * p_ii + ek * G
            gk[:, i] = g * p_ii * d_own + ek * (np.abs(vi) * G + H)
            gw += ek * (np.abs(vi) * G1 + H1)
        else:
            d_own = vi - yi
            gv[:, i] = g * p_ii + ek * G
            gk[:, i] = g * p_ii * d_own + ek * (vi * G - H)
            gw -= ek * (vi * G1 - H1)
        gu += g * p_ii * d_own
        # terms of token i for the sums seen from i - 1
        f = np.exp(shift - logd[:, i])
        yi_t = np.abs(yi) if absolute else yi
        G1 = decay * (G1 + G)
        H1 = decay * (H1 + H)
        G = decay * G + g * f
        H = decay * H + g * yi_t * f
    return gw.sum(axis=0), gu.sum(axis=0), gk, gv


def wkv4_backward_recurrent(w, u, k, v, gy):
    """The four gradients in O(T) by reverse-time sums (any length).

    Same result as ``wkv4_backward_direct`` up to rounding.  Returns
    (gw [C], gu [C], gk [B, T, C], gv [B, T, C]).
    """
    return _wkv4_backward(w, u, k, v, gy, absolute=False)


def wkv4_backward_scale(w, u, k, v, gy):
    """Magnitudes against which rounding errors of the gradients are measured:
    the same sums with every term replaced by its absolute bound.  Each is
    >= the magnitude of the matching gradient.  Returns (gw, gu, gk, gv)."""
    return _wkv4_backward(w, u, k, v, gy, absolute=True)


# ---------------------------------------------------------------------------
# Eagle (RWKV-5) matrix-valued state
# ---------------------------------------------------------------------------

def wkv5_step(S, w, u, r_t, k_t, v_t):
    """One token of the Eagle recurrence.  Returns (o_t, new S).

    [Eagle-Finch] "Eagle": wkv' = s + diag(u) k^T v is read by the
    receptance, then s' = diag(w) s + k^T v.
    S: [B, H, D, D] indexed [key i][value j];  w, u: [H, D];
    r_t, k_t, v_t: [B, H, D].
    o_t[j] = sum_i r_t[i] (S[i, j] + u[i] k_t[i] v_t[j]).
    """
    w, u = _f64(w), _f64(u)
    r_t, k_t, v_t = _f64(r_t), _f64(k_t), _f64(v_t)
    kv = k_t[..., :, None] * v_t[..., None, :]                  # k^T v  [B,H,D,D]
    read = S + u[None, :, :, None] * kv                         # s + diag(u) k^T v
    o_t = np.matmul(r_t[..., None, :], read)[..., 0, :]         # r contracts key i
    S_new = w[None, :, :, None] * S + kv                        # diag(w) s + k^T v
    return o_t, S_new


def wkv5_recurrent(r, k, v, w, u, S0=None):
    """Eagle output over a sequence by the recurrence, state starting at 0.

    r, k, v: [B, T, H, D]; w, u: [H, D].  Returns (o [B, T, H, D], final S).
    """
    r, k, v = _f64(r), _f64(k), _f64(v)
    B, T, H, D = r.shape
    S = np.zeros((B, H, D, D)) if S0 is None else _f64(S0).copy()
    o = np.empty((B, T, H, D))
    for t in range(T):
        o[:, t], S = wkv5_step(S, w, u, r[:, t], k[:, t], v[:, t])
    return o, S


def wkv5_unrolled(r, k, v, w, u):
    """Eagle output as an explicit sum over past tokens (tiny inputs only).

    Unrolling s' = diag(w) s + k^T v from s = 0 gives, at token t,
    s_t[i, j] = sum_{tau < t} w[i]^(t-1-tau) k_tau[i] v_tau[j], so
    o_t[j] = sum_{tau<t} (sum_i r_t[i] w[i]^(t-1-tau) k_tau[i]) v_tau[j]
             + (sum_i r_t[i] u[i] k_t[i]) v_t[j].
    """
    r, k, v, w, u = _f64(r), _f64(k), _f64(v), _f64(w), _f64(u)
    B, T, H, D = r.shape
    o = np.zeros((B, T, H, D))
    for t in range(T):
        for tau in range(t):
            decay = w ** (t - 1 - tau)                          # [H, D]
            coef = (r[:, t] * decay[None] * k[:, tau]).sum(-1)  # [B, H]
            o[:, t] += coef[..., None] * v[:, tau]
        bonus = (r[:, t] * u[None] * k[:, t]).sum(-1)
        o[:, t] += bonus[..., None] * v[:, t]
    return o


def wkv5_scale(r, k, v, w, u):
    """Magnitude bound o_abs >= |o|: the same recurrence on |r|,|k|,|v|,|u|.

    Every term of o is a product of these factors with w in (0, 1], so the
    sum of absolute terms bounds |o| and scales the rounding error.
    """
    o, _ = wkv5_recurrent(np.abs(_f64(r)), np.abs(_f64(k)), np.abs(_f64(v)),
                          w, np.abs(_f64(u)))
    return o


# ---------------------------------------------------------------------------
# Finch (RWKV-6): the Eagle recurrence with a per-token decay w_t
# ---------------------------------------------------------------------------

def wkv6_step(S, w_t, u, r_t, k_t, v_t):
    """One token with its own decay.  w_t, r_t, k_t, v_t: [B, H, D]; u: [H, D].

    [Eagle-Finch] "Finch": the Eagle read-out r (s + diag(u) k^T v), then
    s' = diag(w_t) s + k^T v with this token's decay.
    """
    w_t, u = _f64(w_t), _f64(u)
    r_t, k_t, v_t = _f64(r_t), _f64(k_t), _f64(v_t)
    kv = k_t[..., :, None] * v_t[..., None, :]
    read = S + u[None, :, :, None] * kv
    o_t = np.matmul(r_t[..., None, :], read)[..., 0, :]
    S_new = w_t[..., :, None] * S + kv
    return o_t, S_new


def wkv6_recurrent(r, k, v, w, u, S0=None):
    """Finch output over a sequence by the recurrence.

    r, k, v, w: [B, T, H, D] (w the per-token decay factor); u: [H, D].
    Returns (o [B, T, H, D], final S).
    """
    r, k, v, w = _f64(r), _f64(k), _f64(v), _f64(w)
    B, T, H, D = r.shape
    S = np.zeros((B, H, D, D)) if S0 is None else _f64(S0).copy()
    o = np.empty((B, T, H, D))
    for t in range(T):
        o[:, t], S = wkv6_step(S, w[:, t], u, r[:, t], k[:, t], v[:, t])
    return o, S


def wkv6_unrolled(r, k, v, w, u):
    """Finch output as an explicit sum over past tokens (tiny inputs only).

    Unrolling s_{t+1} = diag(w_t) s_t + k_t^T v_t from s_0 = 0, token
    tau < t reaches s_t scaled by prod_{j=tau+1}^{t-1} w_j (per key channel),
    so o_t[j] = sum_{tau<t} (sum_i r_t[i] prod_j w_j[i] k_tau[i]) v_tau[j]
                + (sum_i r_t[i] u[i] k_t[i]) v_t[j].
    """
    r, k, v, w, u = _f64(r), _f64(k), _f64(v), _f64(w), _f64(u)
    B, T, H, D = r.shape
    o = np.zeros((B, T, H, D))
    for t in range(T):
        for tau in range(t):
            decay = np.prod(w[:, tau + 1:t], axis=1)          # [B, H, D]; empty product = 1
            coef = (r[:, t] * decay * k[:, tau]).sum(-1)        # [B, H]
            o[:, t] += coef[..., None] * v[:, tau]
        bonus = (r[:, t] * u[None] * k[:, t]).sum(-1)
        o[:, t] += bonus[..., None] * v[:, t]
    return o


def wkv6_scale(r, k, v, w, u, S0=None):
    """Magnitude bounds for the tolerance: the same recurrence on |r|, |k|,
    |v|, |u| (and |S0|), w_t being in (0, 1].  Returns (o_abs, S_abs)."""
    return wkv6_recurrent(np.abs(_f64(r)), np.abs(_f64(k)), np.abs(_f64(v)), w,
                          np.abs(_f64(u)), None if S0 is None else np.abs(_f64(S0)))
