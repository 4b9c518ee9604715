"""Bit-exact indexing checks of the matrix-state paths (Eagle and Finch).

[Eagle-Finch] "RWKV-5 Eagle and RWKV-6 Finch", section "Eagle": the state
update s' = diag(w) s + k^T v and the read-out r (s + diag(u) k^T v);
section "Finch": the same with a decay per token.

The inputs (synth.dyadic_matrix_inputs) are sparse one-hot tokens with
power-of-two values and decays of 1, 1/2, 1/4 (Eagle: 1/16 on one head,
2^-16 on another, a growing factor 2 on a third; Finch: 2^-16 on some
tokens), placed across chunk edges and time-segment seams so that
every sum of the exact result has at most one nonzero term.  Every
intermediate of the chunked forms (the decay-scaled bf16 queries and keys,
the score tiles, the bf16 copy of the state) is then an exact power of two,
and a correct kernel returns the float32 rounding of the fp64 oracle bit for
bit.  A wrong chunk offset, a decay power off by one, a key/value transpose
or a seam that drops or repeats a token changes some output by a factor of
two or more, which these tests see, where a tolerance test could not.
"""
import numpy as np
import pytest

import linear_attention_sequence_rwkv_amd as rw
import oracle.wkv_oracle as O
import synth
from wkv_testutil import log, to_dev, torch_dev, tuned

pytestmark = pytest.mark.gpu

B, H = 2, 3


def _seams(T, segs):
    n_chunks = -(-T // 64)
    per = -(-n_chunks // segs)
    return tuple(range(per * 64, T, per * 64))


def _bits(e, name, sl=np.s_[:]):
    torch, _ = torch_dev()
    return to_dev(np.ascontiguousarray(e[name + "_bits"][sl]), torch.bfloat16)


def _assert_bitwise(got, ref64, what):
    ref = np.asarray(ref64, dtype=np.float64).astype(np.float32)
    got = np.asarray(got)
    bad = np.argwhere(got != ref)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements differ; first at {i}: "
                             f"got {got[i]!r}, exact {ref[i]!r}")


def _oracle(e, finch):
    if finch:
        return O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"])
    return O.wkv5_recurrent(e["r"], e["k"], e["v"], e["w"], e["u"])


def _forward(e, finch, sl=np.s_[:], s_in=None):
    torch, _ = torch_dev()
    r, k, v = _bits(e, "r", sl), _bits(e, "k", sl), _bits(e, "v", sl)
    u = to_dev(e["u"])
    if finch:
        wt = to_dev(np.ascontiguousarray(e["wt"][sl]))
        o, s = rw.rwkv_wkv6_forward(r, k, v, wt, u, s_in=s_in, s_out=True)
    else:
        o, s = rw.rwkv_wkv5_forward_state(r, k, v, to_dev(e["w"]), u, s_in=s_in, s_out=True)
    return o, s


def _step(e, finch, s, t):
    sl = np.s_[:, t]
    r, k, v = _bits(e, "r", sl), _bits(e, "k", sl), _bits(e, "v", sl)
    if finch:
        return rw.rwkv_wkv6_step(s, r, k, v, to_dev(np.ascontiguousarray(e["wt"][:, t])),
                                 to_dev(e["u"]))
    return rw.rwkv_wkv5_step(s, r, k, v, to_dev(e["w"]), to_dev(e["u"]))


@pytest.mark.parametrize("dv", [64, 32, 16])
@pytest.mark.parametrize("segs", [1, 2, 3, 4])
def test_eagle_forward_bit_exact(segs, dv):
    torch, _ = torch_dev()
    T = 1100
    seams = _seams(T, segs)
    # one head per path of the kernel: 0 mid-chunk reference, 1 blocks with
    # exact diagonals (2^-16 decays), 2 blocks (1/16 decays), 3 the exact
    # recurrence (a growing row, w = 2)
    H4 = 4
    log(f"dyadic wkv5_forward B={B} T={T} H={H4} segments={segs} value columns={dv} "
        f"seams={seams}")
    e = synth.dyadic_matrix_inputs(B, T, H4, seed=300 + 10 * segs + dv, seams=seams,
                                   slow_head=2, fast_head=1, growing_head=3)
    with tuned(wkv5_segs=segs, wkv5_dv=dv):
        o, s = _forward(e, False)
        torch.cuda.synchronize()
    o_ref, s_ref = _oracle(e, False)
    _assert_bitwise(o.cpu().numpy(), o_ref, "o")
    _assert_bitwise(s.cpu().numpy(), s_ref, "s_out")


@pytest.mark.parametrize("dv", ["64", "32"])
@pytest.mark.parametrize("segs", [1, 2, 3, 4])
def test_finch_forward_bit_exact(segs, dv):
    torch, _ = torch_dev()
    T = 1100
    seams = _seams(T, segs)
    log(f"dyadic wkv6_forward B={B} T={T} H={H} segments={segs} value columns={dv} "
        f"seams={seams}")
    e = synth.dyadic_matrix_inputs(B, T, H, seed=400 + 10 * segs + int(dv), seams=seams,
                                   per_token_decay=True)
    with tuned(wkv6_segs=segs, wkv6_dv=dv):
        o, s = _forward(e, True)
        torch.cuda.synchronize()
    o_ref, s_ref = _oracle(e, True)
    _assert_bitwise(o.cpu().numpy(), o_ref, "o")
    _assert_bitwise(s.cpu().numpy(), s_ref, "s_out")


@pytest.mark.parametrize("finch", [False, True], ids=["eagle", "finch"])
def test_steps_bit_exact(finch):
    """Every token through the single-token step from a zero state."""
    torch, dev = torch_dev()
    T = 200
    log(f"dyadic {'wkv6' if finch else 'wkv5'}_step x{T} B={B} H={H}")
    e = synth.dyadic_matrix_inputs(B, T, H, seed=501 + finch, per_token_decay=finch,
                                   slow_head=None if finch else 1)
    s = torch.zeros((B, H, 64, 64), dtype=torch.float32, device=dev)
    outs = [_step(e, finch, s, t) for t in range(T)]
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=1).cpu().numpy()
    o_ref, s_ref = _oracle(e, finch)
    _assert_bitwise(o, o_ref, "o")
    _assert_bitwise(s.cpu().numpy(), s_ref, "state")


@pytest.mark.parametrize("finch", [False, True], ids=["eagle", "finch"])
@pytest.mark.parametrize("cut", [(129, 7), (64, 1), (300, 33)])
def test_forward_steps_forward_chain_bit_exact(cut, finch):
    """forward(T1) -> N steps -> forward(rest), the state handed on (the last
    hand-over in place), equals one exact pass bit for bit."""
    torch, _ = torch_dev()
    T1, N = cut
    T = 700
    log(f"dyadic {'wkv6' if finch else 'wkv5'} chain T1={T1} steps={N} T={T}")
    e = synth.dyadic_matrix_inputs(B, T, H, seed=600 + T1 + N + finch, per_token_decay=finch,
                                   seams=(T1, T1 + N),
                                   **({} if finch else dict(slow_head=0, fast_head=1,
                                                            growing_head=2)))
    o1, s = _forward(e, finch, np.s_[:, :T1])
    outs = [o1]
    for t in range(T1, T1 + N):
        outs.append(_step(e, finch, s, t)[:, None])
    o3, s3 = _forward(e, finch, np.s_[:, T1 + N:], s_in=s)
    outs.append(o3)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(e, finch)
    _assert_bitwise(torch.cat(outs, dim=1).cpu().numpy(), o_ref, "o")
    _assert_bitwise(s3.cpu().numpy(), s_ref, "final state")
