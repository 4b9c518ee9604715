"""Host-side checks of the kernels' float32 bookkeeping (no GPU).

The RWKV-4 scans carry a history's scale as an anchor: a key kr plus an
integer count n of decay steps since it, n held in a float32
(hist_read_push and hist_concat in csrc/wkv_device.h).  A float32 holds
every integer up to 2^24 and not 2^24 + 1, so a count that passes 2^24
stops advancing and the history stops decaying.  This module replays that
arithmetic in float32 with NumPy and checks that the sequence-length limit
of one call (T <= 2^24 - 64, include/rwkv_wkv.h) keeps every count the
scans can form exact.
"""
import numpy as np

F = np.float32
LIMIT = (1 << 24) - 64


def fma32(a, b, c):
    """fmaf emulated: the float32 product is exact in float64, one rounding
    of the sum to float32 (a second rounding cannot occur for these values)."""
    return F(np.float64(a) * np.float64(b) + np.float64(c))


def read_push(h, k2, v, u2, w2):
    """float32 replay of hist_read_push: returns y and the new (A, Bd, kr, n)."""
    A, Bd, kr, n = h
    base = fma32(-n, w2, F(kr - k2))
    dr, dp = F(base - u2), F(base - w2)
    er, ep = np.exp2(F(-abs(dr))), np.exp2(F(-abs(dp)))
    num = fma32(er, v, A) if dr >= 0 else fma32(er, A, v)
    den = F(Bd + er) if dr >= 0 else fma32(er, Bd, F(1))
    y = F(num / den)
    if dp >= 0:
        return y, (fma32(ep, v, A), F(Bd + ep), kr, F(n + F(1)))
    return y, (fma32(ep, A, v), fma32(ep, Bd, F(1)), F(k2), F(0))


def concat_count(nx, ny):
    """The count hist_concat forms for two histories of nx and ny tokens."""
    return F(F(nx) + F(ny))


def test_count_stalls_past_two_to_the_24():
    """The failure the limit prevents: an anchor kept for more than 2^24
    tokens (a very slow decay after one dominant key) stops counting."""
    w2 = F(2.0 ** -22)
    h = (F(1), F(1), F(50), F((1 << 24) - 3))  # anchored 2^24 - 3 tokens ago
    counts = []
    for _ in range(6):
        _, h = read_push(h, F(0), F(0.5), F(0), w2)
        counts.append(int(h[3]))
    # exact counts would be 2^24 - 2 .. 2^24 + 3
    assert counts[:2] == [(1 << 24) - 2, (1 << 24) - 1]
    assert counts[2:] == [1 << 24] * 4
    # the scale no longer moves: p = kr - n w2 is the same after each token
    p = [fma32(-F(c), w2, F(50)) for c in counts[2:]]
    assert len(set(p)) == 1
    # and a concatenation across the boundary rounds an odd total
    assert int(concat_count((1 << 24) - 10, 137)) != (1 << 24) + 127


def test_counts_stay_exact_within_the_limit():
    """Every count a call can form is at most T plus a few tokens of a block
    (the blocked rescan adds up to 8 to a history's count, and the anchor
    offset a + 1 <= 4): all exact below 2^24 when T <= LIMIT."""
    for n in (LIMIT - 8, LIMIT, LIMIT + 4, LIMIT + 8):
        assert int(F(n)) == n and int(F(F(n) + F(1))) == n + 1
    assert int(concat_count(LIMIT - 128, 128)) == LIMIT
    # the replay keeps counting exactly just below the limit
    h = (F(1), F(1), F(50), F(LIMIT - 8))
    for i in range(8):
        _, h = read_push(h, F(0), F(0.5), F(0), F(2.0 ** -22))
        assert int(h[3]) == LIMIT - 7 + i


def test_replay_matches_the_definition_on_a_short_sequence():
    """The replay itself follows the recurrence it stands for: a few tokens
    from an empty history against the fp64 definition."""
    rng = np.random.default_rng(3)
    k, v = rng.standard_normal(40).astype(F), rng.standard_normal(40).astype(F)
    w, u = F(0.3), F(0.7)
    l2e = F(1.4426950408889634)
    h = (F(0), F(0), F(-1e38), F(0))
    ys = []
    for t in range(40):
        y, h = read_push(h, F(k[t] * l2e), v[t], F(u * l2e), F(w * l2e))
        ys.append(y)
    for t in range(40):
        e = np.array([-(t - 1 - i) * np.float64(w) + k[i] for i in range(t)] + [u + np.float64(k[t])])
        p = np.exp(e - e.max())
        ref = float(np.dot(p, v[:t + 1]) / p.sum())
        assert abs(float(ys[t]) - ref) <= 1e-5 * float(np.dot(p, np.abs(v[:t + 1])) / p.sum())
