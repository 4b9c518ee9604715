"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: a closed
form, a library routine the special case reduces to, an invariant the
mathematics fixes, a hand-worked example, or the other of the pages' two
forms (direct sum vs recurrence; recurrence vs unrolled sum).  The
planted-mistake tests at the end show that plausible slips in the oracle
(an off-by-one decay, a dropped bonus, a flipped sign, a transposed state)
fail at least one pin.
"""
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special

import oracle.wkv_oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _small4(B=2, T=48, C=16, seed=7, **kw):
    return synth.wkv4_inputs(B, T, C, seed, **kw)


def _rel(a, b, scale):
    return float(np.max(np.abs(a - b) / scale))


# ---------------------------------------------------------------- RWKV-4 ---

def direct_vs_recurrent_err(inp):
    yd = O.wkv4_direct(inp["w"], inp["u"], inp["k"], inp["v"])
    yr, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
    S = O.wkv4_scale(inp["w"], inp["u"], inp["k"], inp["v"])
    return _rel(yd, yr, S)


def test_direct_equals_recurrence_tiny_workload():
    inp = synth.wkv4_inputs_for(synth.CFG_WKV4_TINY)
    assert direct_vs_recurrent_err(inp) < 1e-12


def test_direct_equals_recurrence_wide_exponents():
    inp = _small4(omega_lo=-5.0, omega_hi=2.0, u_std=1.0, k_std=3.0)
    assert direct_vs_recurrent_err(inp) < 1e-12


def test_first_token_is_v_exactly():
    inp = _small4(T=1)
    yd = O.wkv4_direct(inp["w"], inp["u"], inp["k"], inp["v"])
    yr, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
    assert np.array_equal(yd, inp["v"].astype(np.float64))
    assert np.array_equal(yr, inp["v"].astype(np.float64))


def test_constant_v_gives_constant_output():
    inp = _small4()
    v = np.full_like(inp["v"], 0.7)
    yr, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], v)
    np.testing.assert_allclose(yr, np.float64(np.float32(0.7)), rtol=1e-14)


def _geometric_den(t, w, u):
    # sum_{j=0}^{t-1} exp(-j w) + exp(u), in closed form
    if t == 0:
        return np.exp(u)
    return (1.0 - np.exp(-t * w)) / (1.0 - np.exp(-w)) + np.exp(u)


@pytest.mark.parametrize("t", [1, 2, 5, 17])
def test_zero_keys_geometric_weights(t):
    """k = 0: the weight of token t-1-j is exp(-j w)/den, den in closed form."""
    C = 5
    w = np.array([0.5, 0.1, 1.3, 2.0, 0.03])
    u = np.array([1.0, -0.4, 0.2, 0.0, 2.5])
    k = np.zeros((1, t + 1, C))
    den = _geometric_den(t, w, u)
    # indicator on the current token
    v = np.zeros((1, t + 1, C))
    v[0, t] = 1.0
    yr, _ = O.wkv4_recurrent(w, u, k, v)
    np.testing.assert_allclose(yr[0, t], np.exp(u) / den, rtol=1e-13)
    # indicator on each past token t-1-j
    for j in range(t):
        v = np.zeros((1, t + 1, C))
        v[0, t - 1 - j] = 1.0
        yr, _ = O.wkv4_recurrent(w, u, k, v)
        np.testing.assert_allclose(yr[0, t], np.exp(-j * w) / den, rtol=1e-13)


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                vals[line[0]] = np.array([float(x) for x in line[1:]])
    return vals


def test_decay_simulator_defaults():
    """The summary page's simulator defaults w=0.5, u=1 over t-4..t."""
    g = _read_golden("wkv4_decay_simulator.txt")
    w, u = g["w"][0], g["u"][0]
    T = len(g["k"])
    k = g["k"].reshape(1, T, 1)
    v = g["v"].reshape(1, T, 1)
    # closed form: past token t-1-j has weight exp(-j w), current exp(u)
    raw = np.array([np.exp(-j * w) for j in range(T - 2, -1, -1)] + [np.exp(u)])
    wts = raw / raw.sum()
    np.testing.assert_allclose(
        wts, [0.045390, 0.074836, 0.123383, 0.203425, 0.552966], atol=5e-7)
    expect = float((wts * g["v"]).sum())
    yd = O.wkv4_direct(np.array([w]), np.array([u]), k, v)
    yr, _ = O.wkv4_recurrent(np.array([w]), np.array([u]), k, v)
    assert abs(yd[0, -1, 0] - expect) < 1e-13
    assert abs(yr[0, -1, 0] - expect) < 1e-13
    assert abs(expect - 4.143740) < 5e-7


def test_zero_decay_is_prefix_softmax():
    """w = 0: y_t = softmax(k_0..k_{t-1}, u+k_t) . v_0..v_t (scipy)."""
    inp = _small4(B=1, T=30, C=6)
    w = np.zeros(6)
    u, k, v = (inp[n].astype(np.float64) for n in ("u", "k", "v"))
    yr, _ = O.wkv4_recurrent(w, u, k, v)
    for t in range(30):
        scores = np.concatenate([k[0, :t], (u + k[0, t])[None]], axis=0)
        p = scipy.special.softmax(scores, axis=0)
        np.testing.assert_allclose(yr[0, t], (p * v[0, : t + 1]).sum(0), rtol=1e-12, atol=1e-14)


def test_huge_decay_is_two_token_softmax():
    """w = 100: only the previous and current tokens matter."""
    inp = _small4(B=1, T=30, C=6)
    w = np.full(6, 100.0)
    u, k, v = (inp[n].astype(np.float64) for n in ("u", "k", "v"))
    yr, _ = O.wkv4_recurrent(w, u, k, v)
    np.testing.assert_array_equal(yr[0, 0], v[0, 0])
    for t in range(1, 30):
        p = scipy.special.softmax(np.stack([k[0, t - 1], u + k[0, t]]), axis=0)
        np.testing.assert_allclose(yr[0, t], p[0] * v[0, t - 1] + p[1] * v[0, t], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("shift", [-80.0, 80.0, 700.0])
def test_key_shift_invariance(shift):
    inp = _small4(k_std=3.0, omega_lo=-5.0, omega_hi=2.0, u_std=1.0)
    y0, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
    y1, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"].astype(np.float64) + shift, inp["v"])
    S = O.wkv4_scale(inp["w"], inp["u"], inp["k"], inp["v"])
    assert _rel(y0, y1, S) < 1e-12


def test_value_affine_equivariance():
    inp = _small4()
    a, b = -2.5, 3.25
    y0, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
    y1, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], a * inp["v"].astype(np.float64) + b)
    np.testing.assert_allclose(y1, a * y0 + b, rtol=1e-12, atol=1e-12)


def test_convex_hull_and_scale_bound():
    inp = _small4(k_std=3.0)
    v = inp["v"].astype(np.float64)
    y, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], v)
    lo = np.minimum.accumulate(v, axis=1)
    hi = np.maximum.accumulate(v, axis=1)
    assert np.all(y >= lo - 1e-12) and np.all(y <= hi + 1e-12)
    S = O.wkv4_scale(inp["w"], inp["u"], inp["k"], v)
    assert np.all(np.abs(y) <= S * (1 + 1e-12))


def test_split_sequence_equals_whole():
    inp = _small4(T=64)
    w, u, k, v = inp["w"], inp["u"], inp["k"], inp["v"]
    y_all, st_all = O.wkv4_recurrent(w, u, k, v)
    y1, st = O.wkv4_recurrent(w, u, k[:, :23], v[:, :23])
    y2, st2 = O.wkv4_recurrent(w, u, k[:, 23:], v[:, 23:], state=st)
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), y_all, rtol=1e-13, atol=1e-14)
    m_a, l_a = O.wkv4_canonical_state(st_all)
    m_b, l_b = O.wkv4_canonical_state(st2)
    np.testing.assert_allclose(m_a, m_b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l_a, l_b, rtol=1e-13)


def test_final_state_is_the_decayed_history():
    """State after T tokens: a/b = weighted mean of v with log-weights
    k_i - (T-1-i) w, and log b = logsumexp of those log-weights."""
    inp = _small4(T=40, k_std=3.0)
    w, u = inp["w"].astype(np.float64), inp["u"]
    k, v = inp["k"].astype(np.float64), inp["v"].astype(np.float64)
    _, st = O.wkv4_recurrent(w, u, k, v)
    mean, logden = O.wkv4_canonical_state(st)
    T = k.shape[1]
    lw = k - (T - 1 - np.arange(T))[None, :, None] * w[None, None, :]
    np.testing.assert_allclose(logden, scipy.special.logsumexp(lw, axis=1), rtol=1e-13)
    p = scipy.special.softmax(lw, axis=1)
    np.testing.assert_allclose(mean, (p * v).sum(1), rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------- Eagle ---

def _small5(B=2, T=20, H=2, D=8, seed=11, **kw):
    return synth.wkv5_inputs(B, T, H, D, seed, **kw)


def recurrent_vs_unrolled_err(inp):
    o_r, _ = O.wkv5_recurrent(inp["r"], inp["k"], inp["v"], inp["w"], inp["u"])
    o_u = O.wkv5_unrolled(inp["r"], inp["k"], inp["v"], inp["w"], inp["u"])
    sc = O.wkv5_scale(inp["r"], inp["k"], inp["v"], inp["w"], inp["u"])
    return _rel(o_r, o_u, sc + 1e-300)


def test_eagle_recurrence_equals_unrolled_sum():
    assert recurrent_vs_unrolled_err(_small5()) < 1e-12
    assert recurrent_vs_unrolled_err(_small5(omega_lo=-1.0, omega_hi=2.0)) < 1e-12


def test_eagle_no_decay_is_masked_matmul():
    """w = 1: o = (strict_lower(R K^T) + diag(beta)) V per (b, h)."""
    inp = _small5(T=24, D=16)
    r, k, v = (inp[n].astype(np.float64) for n in ("r", "k", "v"))
    u = inp["u"].astype(np.float64)
    w = np.ones_like(u)
    o, _ = O.wkv5_recurrent(r, k, v, w, u)
    B, T, H, D = r.shape
    for b in range(B):
        for h in range(H):
            R, K, V = r[b, :, h], k[b, :, h], v[b, :, h]
            A = np.tril(R @ K.T, -1) + np.diag((R * u[h] * K).sum(-1))
            np.testing.assert_allclose(o[b, :, h], A @ V, rtol=1e-12, atol=1e-15)


def test_eagle_single_channel_is_iir_filter():
    """D = 1: s_t = sum_{tau<t} w^(t-1-tau) k_tau v_tau is a first-order IIR
    filter of x = k v (scipy.signal.lfilter), read one step late."""
    rng = np.random.default_rng(5)
    T = 50
    r, k, v = (rng.standard_normal((1, T, 1, 1)) for _ in range(3))
    w = np.array([[0.83]])
    u = np.array([[0.6]])
    o, _ = O.wkv5_recurrent(r, k, v, w, u)
    x = (k * v)[0, :, 0, 0]
    incl = scipy.signal.lfilter([1.0], [1.0, -w[0, 0]], x)   # sum_{m<=n} w^(n-m) x_m
    s = np.concatenate([[0.0], incl[:-1]])
    expect = r[0, :, 0, 0] * (s + u[0, 0] * x)
    np.testing.assert_allclose(o[0, :, 0, 0], expect, rtol=1e-12, atol=1e-15)


def test_eagle_hand_worked_orientation():
    """Dyadic example with D=2 that separates key rows from value columns.

    Token 0: k = e0, v = e1, so s gains s[0][1] = 1 (key 0, value 1).
    Tokens 1 and 2 read with r = e0 and add nothing (k = 0).
    o_1 = s[0, :] = (0, 1); then s decays by diag(w): o_2 = (0, w[0]).
    Token 0 itself reads u[0] * k0[0] * v0 = (0, u[0]).
    """
    w = np.array([[0.5, 0.25]])
    u = np.array([[2.0, 4.0]])
    r = np.zeros((1, 3, 1, 2)); r[0, :, 0, 0] = 1.0
    k = np.zeros((1, 3, 1, 2)); k[0, 0, 0, 0] = 1.0
    v = np.zeros((1, 3, 1, 2)); v[0, 0, 0, 1] = 1.0
    o, S = O.wkv5_recurrent(r, k, v, w, u)
    np.testing.assert_array_equal(o[0, :, 0], [[0.0, 2.0], [0.0, 1.0], [0.0, 0.5]])
    np.testing.assert_array_equal(S[0, 0], [[0.0, 0.25], [0.0, 0.0]])


def test_eagle_linearity_and_bound():
    inp = _small5()
    r, k, v = (inp[n].astype(np.float64) for n in ("r", "k", "v"))
    w, u = inp["w"], inp["u"]
    o, _ = O.wkv5_recurrent(r, k, v, w, u)
    o2, _ = O.wkv5_recurrent(r, k, 3.0 * v - 0.5 * r, w, u)
    o3, _ = O.wkv5_recurrent(r, k, r, w, u)
    np.testing.assert_allclose(o2, 3.0 * o - 0.5 * o3, rtol=1e-11, atol=1e-14)
    o4, _ = O.wkv5_recurrent(-2.0 * r, k, v, w, u)
    np.testing.assert_allclose(o4, -2.0 * o, rtol=1e-13, atol=1e-16)
    sc = O.wkv5_scale(r, k, v, w, u)
    assert np.all(np.abs(o) <= sc * (1 + 1e-12) + 1e-300)


def test_eagle_split_sequence():
    inp = _small5(T=30)
    r, k, v, w, u = (inp[n] for n in ("r", "k", "v", "w", "u"))
    o_all, S_all = O.wkv5_recurrent(r, k, v, w, u)
    o1, S1 = O.wkv5_recurrent(r[:, :13], k[:, :13], v[:, :13], w, u)
    o2, S2 = O.wkv5_recurrent(r[:, 13:], k[:, 13:], v[:, 13:], w, u, S0=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o_all, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(S2, S_all, rtol=1e-13, atol=1e-16)


# ------------------------------------------------- RWKV-4 backward pins ---

def _grad_case(B=2, T=24, C=6, seed=11, **kw):
    inp = synth.wkv4_inputs(B, T, C, seed, **kw)
    gy = synth.rng_for(seed + 100).standard_normal((B, T, C))
    return inp, gy


def _grads(fn, inp, gy):
    return fn(inp["w"], inp["u"], inp["k"], inp["v"], gy)


@pytest.mark.parametrize("kw", [{}, {"k_std": 3.0, "omega_lo": -5.0, "omega_hi": 2.0},
                                {"omega_lo": -8.0, "omega_hi": -6.0}])
def test_backward_direct_equals_recurrence(kw):
    inp, gy = _grad_case(**kw)
    d = _grads(O.wkv4_backward_direct, inp, gy)
    r = _grads(O.wkv4_backward_recurrent, inp, gy)
    sc = _grads(O.wkv4_backward_scale, inp, gy)
    for a, b, m in zip(d, r, sc):
        assert _rel(a, b, m) < 1e-12


def test_backward_key_shift_is_harmless():
    inp, gy = _grad_case()
    ref = _grads(O.wkv4_backward_recurrent, inp, gy)
    shifted = _grads(O.wkv4_backward_recurrent, dict(inp, k=inp["k"].astype(np.float64) + 80.0),
                     gy)
    sc = _grads(O.wkv4_backward_scale, inp, gy)
    for a, b, m in zip(ref, shifted, sc):
        assert _rel(a, b, m) < 1e-10


def test_backward_matches_finite_differences():
    """Central differences of the direct forward sum, every input scalar."""
    inp, gy = _grad_case(B=1, T=7, C=3, seed=5)
    args = {n: np.asarray(inp[n], np.float64) for n in ("w", "u", "k", "v")}

    def loss(a):
        return float((O.wkv4_direct(a["w"], a["u"], a["k"], a["v"]) * gy).sum())

    gw, gu, gk, gv = O.wkv4_backward_direct(args["w"], args["u"], args["k"], args["v"], gy)
    h = 1e-6
    for name, g in (("w", gw), ("u", gu), ("k", gk), ("v", gv)):
        fd = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            plus = {n: a.copy() for n, a in args.items()}
            minus = {n: a.copy() for n, a in args.items()}
            plus[name][idx] += h
            minus[name][idx] -= h
            fd[idx] = (loss(plus) - loss(minus)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_matches_autograd_of_the_definition():
    """float64 autograd through an independent torch transcription of WKV_t."""
    torch = pytest.importorskip("torch")
    inp, gy = _grad_case(B=2, T=12, C=4, seed=9)
    w, u, k, v = (torch.tensor(np.asarray(inp[n], np.float64), requires_grad=True)
                  for n in ("w", "u", "k", "v"))
    T = k.shape[1]
    ys = []
    for t in range(T):
        age = torch.arange(t - 1, -1, -1, dtype=torch.float64)[None, :, None]
        logits = torch.cat([k[:, :t] - age * w, (u + k[:, t])[:, None]], dim=1)
        ys.append((torch.softmax(logits, dim=1) * v[:, :t + 1]).sum(dim=1))
    (torch.stack(ys, dim=1) * torch.tensor(gy)).sum().backward()
    got = O.wkv4_backward_direct(inp["w"], inp["u"], inp["k"], inp["v"], gy)
    for g, t_ in zip(got, (w, u, k, v)):
        np.testing.assert_allclose(g, t_.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_backward_invariants():
    inp, gy = _grad_case(T=30)
    gw, gu, gk, gv = _grads(O.wkv4_backward_recurrent, inp, gy)
    # y is unchanged by k -> k + c and moves by b under v -> v + b
    np.testing.assert_allclose(gk.sum(axis=1), 0.0, atol=1e-11)
    np.testing.assert_allclose(gv.sum(axis=1), gy.sum(axis=1), rtol=1e-11, atol=1e-12)
    # a single token: y = v whatever w, u, k
    one = {n: (inp[n][:, :1] if n in ("k", "v") else inp[n]) for n in inp}
    gw1, gu1, gk1, gv1 = _grads(O.wkv4_backward_recurrent, one, gy[:, :1])
    assert np.all(gw1 == 0) and np.all(gu1 == 0) and np.all(gk1 == 0)
    np.testing.assert_allclose(gv1, gy[:, :1], rtol=1e-15)


def test_backward_scale_bounds_every_gradient():
    inp, gy = _grad_case(k_std=3.0)
    got = _grads(O.wkv4_backward_recurrent, inp, gy)
    sc = _grads(O.wkv4_backward_scale, inp, gy)
    for g, m in zip(got, sc):
        assert np.all(np.abs(g) <= m * (1 + 1e-12) + 1e-300)


# ------------------------------------------------------------ Finch pins ---

def _small6(B=2, T=11, H=3, D=5, seed=13, **kw):
    return synth.wkv6_inputs(B, T, H, D, seed, **kw)


def _finch_err(e):
    o1, _ = O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"])
    o2 = O.wkv6_unrolled(e["r"], e["k"], e["v"], e["wt"], e["u"])
    o_abs, _ = O.wkv6_scale(e["r"], e["k"], e["v"], e["wt"], e["u"])
    return _rel(o1, o2, o_abs)


def test_finch_recurrence_equals_unrolled_sum():
    assert _finch_err(_small6()) < 1e-13
    assert _finch_err(_small6(delta_std=2.0, seed=3)) < 1e-13


def test_finch_with_constant_decay_is_eagle():
    e = _small6()
    wt = np.broadcast_to(e["w"][None, None], e["wt"].shape)
    o6, S6 = O.wkv6_recurrent(e["r"], e["k"], e["v"], wt, e["u"])
    o5, S5 = O.wkv5_recurrent(e["r"], e["k"], e["v"], e["w"], e["u"])
    np.testing.assert_array_equal(o6, o5)
    np.testing.assert_array_equal(S6, S5)


def test_finch_no_decay_single_channel_is_a_prefix_sum():
    rng = np.random.default_rng(4)
    T = 40
    r, k, v = (rng.standard_normal((1, T, 1, 1)) for _ in range(3))
    u = np.array([[0.3]])
    o, _ = O.wkv6_recurrent(r, k, v, np.ones((1, T, 1, 1)), u)
    kv = (k * v)[0, :, 0, 0]
    hist = np.concatenate([[0.0], np.cumsum(kv)[:-1]])
    np.testing.assert_allclose(o[0, :, 0, 0], r[0, :, 0, 0] * (hist + 0.3 * kv), rtol=1e-13)


def test_finch_hand_worked_decay_timing():
    """D=1, u=0: s1 = k0 v0 = 1, s2 = w1 s1 + k1 v1 = 0.25 + 2 = 2.25.  The
    first token's decay w0 multiplies the empty state and cannot matter; the
    second token's decay w1 = 0.25 is the one applied to s1."""
    r = np.ones((1, 3, 1, 1))
    k = np.array([1.0, 2.0, 0.5]).reshape(1, 3, 1, 1)
    v = np.array([1.0, 1.0, 2.0]).reshape(1, 3, 1, 1)
    w = np.array([0.5, 0.25, 0.125]).reshape(1, 3, 1, 1)
    o, S = O.wkv6_recurrent(r, k, v, w, np.zeros((1, 1)))
    np.testing.assert_array_equal(o[0, :, 0, 0], [0.0, 1.0, 2.25])
    np.testing.assert_array_equal(S[0, 0], [[0.125 * 2.25 + 1.0]])


def test_finch_split_sequence():
    e = _small6(T=20)
    args = [e[n] for n in ("r", "k", "v", "wt")]
    o_all, S_all = O.wkv6_recurrent(*args, e["u"])
    o1, S1 = O.wkv6_recurrent(*(a[:, :7] for a in args), e["u"])
    o2, S2 = O.wkv6_recurrent(*(a[:, 7:] for a in args), e["u"], S0=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o_all, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(S2, S_all, rtol=1e-13, atol=1e-16)


def test_finch_scale_bounds_output():
    e = _small6(delta_std=1.0)
    o, S = O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"])
    o_abs, S_abs = O.wkv6_scale(e["r"], e["k"], e["v"], e["wt"], e["u"])
    assert np.all(np.abs(o) <= o_abs * (1 + 1e-12)) and np.all(np.abs(S) <= S_abs * (1 + 1e-12))


# ------------------------------------------------------- planted mistakes ---

_WKV4_STEP = O.wkv4_step


def _mut_decay_off_by_one(state, w, u, k_t, v_t):
    # decay applied to the history before it is read (one step too early)
    num, den, ref = state
    return _WKV4_STEP((num, den, ref - np.asarray(w, float)), w, u, k_t, v_t)


def _mut_no_bonus(state, w, u, k_t, v_t):
    return _WKV4_STEP(state, w, np.zeros_like(np.asarray(u, float)), k_t, v_t)


def _mut_sign_w(state, w, u, k_t, v_t):
    return _WKV4_STEP(state, -np.asarray(w, float), u, k_t, v_t)


@pytest.mark.parametrize("mutant", [_mut_decay_off_by_one, _mut_no_bonus, _mut_sign_w])
def test_pins_catch_planted_wkv4_mistakes(monkeypatch, mutant):
    monkeypatch.setattr(O, "wkv4_step", mutant)
    inp = synth.wkv4_inputs_for(synth.CFG_WKV4_TINY)
    yd = O.wkv4_direct(inp["w"], inp["u"], inp["k"], inp["v"])
    yr, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
    assert np.max(np.abs(yd - yr)) > 1e-3


def test_pins_catch_planted_backward_mistake(monkeypatch):
    # a forward without the bonus inside the reverse-time evaluation
    monkeypatch.setattr(O, "wkv4_step", _mut_no_bonus)
    inp, gy = _grad_case()
    d = _grads(O.wkv4_backward_direct, inp, gy)
    r = _grads(O.wkv4_backward_recurrent, inp, gy)
    assert max(float(np.max(np.abs(a - b))) for a, b in zip(d, r)) > 1e-3


def test_pins_catch_transposed_eagle_state(monkeypatch):
    def transposed(S, w, u, r_t, k_t, v_t):
        # the receptance contracts the value index of the history
        o, _ = original(np.swapaxes(S, -1, -2), w, u, r_t, k_t, v_t)
        _, S2 = original(S, w, u, r_t, k_t, v_t)
        return o, S2
    original = O.wkv5_step
    monkeypatch.setattr(O, "wkv5_step", transposed)
    assert recurrent_vs_unrolled_err(_small5()) > 1e-3


def test_pins_catch_eagle_decay_on_value_index(monkeypatch):
    def value_decay(S, w, u, r_t, k_t, v_t):
        o, _ = original(S, w, u, r_t, k_t, v_t)
        kv = np.asarray(k_t, float)[..., :, None] * np.asarray(v_t, float)[..., None, :]
        return o, np.asarray(w, float)[None, :, None, :] * S + kv
    original = O.wkv5_step
    monkeypatch.setattr(O, "wkv5_step", value_decay)
    assert recurrent_vs_unrolled_err(_small5()) > 1e-3


def test_pins_catch_finch_decay_after_adding(monkeypatch):
    def decay_after(S, w_t, u, r_t, k_t, v_t):
        # the token's own k^T v decayed by its own w_t
        o, _ = original(S, w_t, u, r_t, k_t, v_t)
        kv = np.asarray(k_t, float)[..., :, None] * np.asarray(v_t, float)[..., None, :]
        return o, np.asarray(w_t, float)[..., :, None] * (S + kv)
    original = O.wkv6_step
    monkeypatch.setattr(O, "wkv6_step", decay_after)
    assert _finch_err(_small6()) > 1e-3
