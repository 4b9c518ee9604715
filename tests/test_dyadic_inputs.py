"""The one-hot dyadic inputs behind the bit-exact GPU tests, checked on the
CPU: every exact result is a power of two (or zero) in the normal float32
range, so float32 rounding is exact; and plausible indexing mistakes,
planted in a copy of the oracle's recurrence, change the float32 bits.
Without the second property the bitwise GPU tests would prove nothing."""
import numpy as np
import pytest

import oracle.wkv_oracle as O
import synth


def _powers_of_two(x):
    """Every exact value is 0, a power of two in the normal float32 range, or
    so small (<= 2^-151, a write decayed long ago) that float32 holds 0."""
    x = np.asarray(x, dtype=np.float64)
    nz = x[x != 0]
    m, _ = np.frexp(np.abs(nz))
    assert np.all(m == 0.5), "a result is not a power of two"
    tiny = np.abs(nz) <= 2.0 ** -151
    assert np.all(tiny | (np.abs(nz) >= 2.0 ** -126)), "a result is subnormal in float32"
    kept = np.where(np.abs(x) <= 2.0 ** -151, 0.0, x)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), kept)
    return int((~tiny).sum())


def _mutant(r, k, v, w, u, kind, per_token):
    """A copy of the Eagle/Finch recurrence with one planted mistake."""
    r, k, v, w, u = (np.asarray(a, dtype=np.float64) for a in (r, k, v, w, u))
    B, T, H, D = r.shape
    S = np.zeros((B, H, D, D))
    o = np.empty((B, T, H, D))
    for t in range(T):
        wt = w[:, t] if per_token else w[None]
        kv = k[:, t, :, :, None] * v[:, t, :, None, :]
        if kind == "decay_before_read":      # the state decays before it is read
            S = wt[..., None] * S
        read = S + (0 if kind == "no_bonus" else u[None, :, :, None] * kv)
        if kind == "transposed":             # r contracts the value index
            read = np.swapaxes(read, -1, -2)
        o[:, t] = np.matmul(r[:, t, :, None, :], read)[..., 0, :]
        if kind == "decay_before_read":
            S = S + kv
        elif kind == "value_decay":          # decay on value columns
            S = wt[..., None, :] * S + kv
        else:
            S = wt[..., None] * S + kv
    return o


@pytest.mark.parametrize("per_token", [False, True], ids=["eagle", "finch"])
def test_exact_results_are_float32_powers_of_two(per_token):
    # Eagle: head 0 all decays in {1, 1/2, 1/4}, head 1 some 2^-16, head 2
    # some 1/16, head 3 one growing row (factor 2)
    H = 3 if per_token else 4
    e = synth.dyadic_matrix_inputs(2, 1100, H, seed=11, per_token_decay=per_token,
                                   seams=(320, 640, 960),
                                   **({} if per_token else
                                      dict(slow_head=2, fast_head=1, growing_head=3)))
    if per_token:
        o, S = O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"])
    else:
        o, S = O.wkv5_recurrent(e["r"], e["k"], e["v"], e["w"], e["u"])
    n_o = _powers_of_two(o)
    n_s = _powers_of_two(S)
    # dense enough to exercise every path: many nonzero outputs and states
    assert n_o > 500 and n_s > 100
    if not per_token:
        # the special rows are written and read: outputs that are the
        # product of a 2^-16 decay, and of a factor 2 (w^d with d >= 1)
        for h, kind_w in ((1, 2.0 ** -16), (3, 2.0)):
            rows = np.flatnonzero(e["w"][h] == kind_w)
            assert rows.size > 0
            read = np.abs(e["r"][:, :, h][..., rows]).sum(-1) > 0
            wrote_before = np.cumsum(np.abs(e["k"][:, :, h][..., rows]).sum(-1) > 0, axis=1) > 0
            assert np.any(read & wrote_before & (np.abs(o[:, :, h]).sum(-1) > 0))


@pytest.mark.parametrize("per_token", [False, True], ids=["eagle", "finch"])
@pytest.mark.parametrize("kind", ["decay_before_read", "no_bonus", "transposed", "value_decay"])
def test_planted_mistakes_change_the_bits(kind, per_token):
    e = synth.dyadic_matrix_inputs(2, 300, 3, seed=12, per_token_decay=per_token,
                                   slow_head=None if per_token else 1)
    w = e["wt"] if per_token else e["w"]
    if per_token:
        ref, _ = O.wkv6_recurrent(e["r"], e["k"], e["v"], w, e["u"])
    else:
        ref, _ = O.wkv5_recurrent(e["r"], e["k"], e["v"], w, e["u"])
    bad = _mutant(e["r"], e["k"], e["v"], w, e["u"], kind, per_token)
    assert not np.array_equal(bad.astype(np.float32), ref.astype(np.float32))


def test_token_shift_changes_the_bits():
    """An output one token late (a chunk or seam offset slip) is caught."""
    e = synth.dyadic_matrix_inputs(1, 300, 2, seed=13, seams=(128,))
    ref, _ = O.wkv5_recurrent(e["r"], e["k"], e["v"], e["w"], e["u"])
    shifted = np.concatenate([np.zeros_like(ref[:, :1]), ref[:, :-1]], axis=1)
    assert not np.array_equal(shifted.astype(np.float32), ref.astype(np.float32))
