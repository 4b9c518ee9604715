"""GPU parity against the fp64 oracle on shapes drawn at random (fixed seed):
the RWKV-4 forward and backward, and the Eagle and Finch forwards, each with
random sizes that land anywhere relative to the tiles, channel blocks,
chunks and time segments, and with random plan overrides (value slices,
segment counts) where the operator has them.  Tolerances as in the
per-operator tests: 1e-4 of the magnitude scale for RWKV-4, 2e-2 of o_abs
for the bf16-MFMA forwards."""
import numpy as np
import pytest

import linear_attention_sequence_rwkv_amd as rw
import oracle.wkv_oracle as O
import synth
from wkv_testutil import (WKV4_TOL, WKV5_TOL, log, to_dev, torch_dev, tuned, wkv4_scaled_err,
                          wkv5_scaled_err)

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261203)


def _draw(n, lo_hi):
    return [tuple(int(_rng.integers(lo, hi + 1)) for lo, hi in lo_hi) for _ in range(n)]


WKV4_FWD = _draw(10, [(1, 4), (1, 2600), (1, 320)])
WKV4_BWD = _draw(8, [(1, 3), (1, 1500), (1, 200)])
WKV5 = [s + (int(_rng.choice([64, 32, 16])), int(_rng.integers(0, 5)))
        for s in _draw(8, [(1, 2), (1, 700), (1, 3)])]
WKV6 = [s + (int(_rng.choice([64, 32])), int(_rng.integers(0, 5)))
        for s in _draw(8, [(1, 2), (1, 700), (1, 3)])]


@pytest.mark.parametrize("shape", WKV4_FWD)
def test_wkv4_forward(shape):
    torch, _ = torch_dev()
    B, T, C = shape
    omega_hi = 3.0 if (B + T + C) % 2 else 1.0
    log(f"wkv4_forward B={B} T={T} C={C} omega_hi={omega_hi}")
    e = synth.wkv4_inputs(B, T, C, seed=B * 100003 + T * 331 + C, omega_hi=omega_hi)
    y = rw.rwkv_wkv4_forward(*(to_dev(e[n]) for n in ("w", "u", "k", "v")))
    torch.cuda.synchronize()
    y_ref, _ = O.wkv4_recurrent(e["w"], e["u"], e["k"], e["v"])
    err = wkv4_scaled_err(y.cpu().numpy(), y_ref, O.wkv4_scale(e["w"], e["u"], e["k"], e["v"]))
    log(f"  err={err:.2e}")
    assert err <= WKV4_TOL


@pytest.mark.parametrize("shape", WKV4_BWD)
def test_wkv4_backward(shape):
    torch, _ = torch_dev()
    B, T, C = shape
    log(f"wkv4_backward B={B} T={T} C={C}")
    e = synth.wkv4_backward_inputs(B, T, C, seed=B * 100003 + T * 331 + C + 7)
    args = [e[n] for n in ("w", "u", "k", "v", "gy")]
    got = rw.rwkv_wkv4_backward(*(to_dev(a) for a in args))
    torch.cuda.synchronize()
    ref = O.wkv4_backward_recurrent(*args)
    scale = O.wkv4_backward_scale(*args)
    for name, g, r, s in zip(("gw", "gu", "gk", "gv"), got, ref, scale):
        g = g.cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(g - r) / np.maximum(s, 1e-30))) if g.size else 0.0
        log(f"  {name}={err:.2e}")
        assert err <= WKV4_TOL, name
        assert np.all(np.isfinite(g))


@pytest.mark.parametrize("case", WKV5)
def test_eagle_forward(case):
    torch, _ = torch_dev()
    B, T, H, dv, segs = case
    omega_hi = 2.0 if T % 2 else 0.0
    log(f"wkv5_forward B={B} T={T} H={H} value slice {dv} segments {segs or 'default'} "
        f"omega_hi={omega_hi}")
    e = synth.wkv5_inputs(B, T, H, 64, seed=B * 1009 + T * 31 + H, omega_hi=omega_hi)
    with tuned(wkv5_dv=dv, wkv5_segs=segs or None):
        o = rw.rwkv_wkv5_forward(to_dev(e["r_bits"], torch.bfloat16),
                                 to_dev(e["k_bits"], torch.bfloat16),
                                 to_dev(e["v_bits"], torch.bfloat16),
                                 to_dev(e["w"]), to_dev(e["u"]))
        torch.cuda.synchronize()
    o_ref, _ = O.wkv5_recurrent(e["r"], e["k"], e["v"], e["w"], e["u"])
    err = wkv5_scaled_err(o.cpu().numpy(), o_ref,
                          O.wkv5_scale(e["r"], e["k"], e["v"], e["w"], e["u"]))
    log(f"  err={err:.3e}")
    assert err <= WKV5_TOL


@pytest.mark.parametrize("case", WKV6)
def test_finch_forward(case):
    torch, _ = torch_dev()
    B, T, H, dv, segs = case
    delta_std = 1.0 if T % 2 else 0.5
    log(f"wkv6_forward B={B} T={T} H={H} value slice {dv} segments {segs or 'default'} "
        f"delta_std={delta_std}")
    e = synth.wkv6_inputs(B, T, H, 64, seed=B * 1009 + T * 31 + H + 5, delta_std=delta_std)
    with tuned(wkv6_dv=dv, wkv6_segs=segs or None):
        o, _ = rw.rwkv_wkv6_forward(to_dev(e["r_bits"], torch.bfloat16),
                                    to_dev(e["k_bits"], torch.bfloat16),
                                    to_dev(e["v_bits"], torch.bfloat16), to_dev(e["wt"]),
                                    to_dev(e["u"]))
        torch.cuda.synchronize()
    o_ref, _ = O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"])
    o_abs, _ = O.wkv6_scale(e["r"], e["k"], e["v"], e["wt"], e["u"])
    err = wkv5_scaled_err(o.cpu().numpy(), o_ref, o_abs)
    log(f"  err={err:.3e}")
    assert err <= WKV5_TOL
