"""GPU parity of the Eagle (RWKV-5) forward against the fp64 oracle.

Tolerance: max |o_gpu - o_oracle| / o_abs <= 2e-2, where o_abs is the same
recurrence over |r|, |k|, |v|, |u| (a bound on |o| that scales the rounding
error of bf16 products with float32 accumulation).
"""
import os

import numpy as np
import pytest

import linear_attention_sequence_rwkv_amd as rw
import oracle.wkv_oracle as O
import synth
from wkv_testutil import WKV5_TOL, log, to_dev, torch_dev, wkv5_scaled_err

pytestmark = pytest.mark.gpu


def gpu_wkv5(inp, dv=None):
    torch, _ = torch_dev()
    old = os.environ.get("RWKV_WKV5_DV")
    if dv is not None:
        os.environ["RWKV_WKV5_DV"] = str(dv)
    try:
        o = rw.rwkv_wkv5_forward(to_dev(inp["r_bits"], torch.bfloat16),
                                 to_dev(inp["k_bits"], torch.bfloat16),
                                 to_dev(inp["v_bits"], torch.bfloat16),
                                 to_dev(inp["w"]), to_dev(inp["u"]))
        torch.cuda.synchronize()
    finally:
        if dv is not None:
            if old is None:
                del os.environ["RWKV_WKV5_DV"]
            else:
                os.environ["RWKV_WKV5_DV"] = old
    return o.cpu().numpy()


def oracle_wkv5(inp, b_idx=None, h_idx=None):
    r, k, v, w, u = (inp[n] for n in ("r", "k", "v", "w", "u"))
    if b_idx is not None:
        r, k, v = r[b_idx], k[b_idx], v[b_idx]
    if h_idx is not None:
        r, k, v, w, u = r[:, :, h_idx], k[:, :, h_idx], v[:, :, h_idx], w[h_idx], u[h_idx]
    o, _ = O.wkv5_recurrent(r, k, v, w, u)
    return o, O.wkv5_scale(r, k, v, w, u)


@pytest.mark.parametrize("dv", [32, 16])
@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 100, 3), (1, 257, 2), (3, 64, 1), (2, 200, 9)])
def test_small_shapes(shape, dv):
    B, T, H = shape
    log(f"wkv5_forward B={B} T={T} H={H} D=64 value slice {dv}")
    inp = synth.wkv5_inputs(B, T, H, 64, seed=40 + T)
    o = gpu_wkv5(inp, dv)
    o_ref, o_abs = oracle_wkv5(inp)
    err = wkv5_scaled_err(o, o_ref, o_abs)
    log(f"  err={err:.3e}")
    assert err <= WKV5_TOL


def test_eagle_workload_sampled_heads():
    """B=4 T=4096 H=32 D=64 on the GPU; the oracle runs 2 batches x 4 heads."""
    cfg = synth.CFG_WKV5_EAGLE
    log(f"wkv5_forward {cfg.name} seed={cfg.seed} (oracle on sampled heads)")
    inp = synth.wkv5_inputs_for(cfg)
    o = gpu_wkv5(inp)
    bs, hs = np.array([0, 3]), np.array([0, 7, 19, 31])
    o_ref, o_abs = oracle_wkv5(inp, bs, hs)
    err = wkv5_scaled_err(o[bs][:, :, hs], o_ref, o_abs)
    log(f"  err={err:.3e}")
    assert err <= WKV5_TOL
    assert np.all(np.isfinite(o))


@pytest.mark.parametrize("dv", [32, 16])
def test_no_decay_and_fast_decay_extremes(dv):
    B, T, H = 1, 300, 2
    inp = synth.wkv5_inputs(B, T, H, 64, seed=77)
    for name, wv in (("w=1", 1.0), ("w=0.05", 0.05)):
        log(f"wkv5_forward {name} value slice {dv}")
        case = dict(inp, w=np.full((H, 64), wv, np.float32))
        o = gpu_wkv5(case, dv)
        o_ref, o_abs = oracle_wkv5(case)
        assert wkv5_scaled_err(o, o_ref, o_abs) <= WKV5_TOL, name
