"""GPU parity of the Finch (per-token decay) forward and step against the
fp64 oracle.

Tolerance as for Eagle: max |o - o_ref| / o_abs <= 2e-2 for the bf16-MFMA
forward (o_abs: the same recurrence over |r|, |k|, |v|, |u|); the step is
exact float32 arithmetic on the bf16 inputs (1e-5).
"""
import numpy as np
import pytest

import linear_attention_sequence_rwkv_amd as rw
import oracle.wkv_oracle as O
import synth
from wkv_testutil import WKV5_TOL, log, to_dev, torch_dev, tuned, wkv5_scaled_err

pytestmark = pytest.mark.gpu


def _bits(e, name, sl=np.s_[:]):
    torch, _ = torch_dev()
    return to_dev(np.ascontiguousarray(e[name + "_bits"][sl]), torch.bfloat16)


def gpu_finch(e, s_in=None, s_out=None):
    torch, _ = torch_dev()
    o, s = rw.rwkv_wkv6_forward(_bits(e, "r"), _bits(e, "k"), _bits(e, "v"), to_dev(e["wt"]),
                                to_dev(e["u"]), s_in=s_in, s_out=s_out)
    torch.cuda.synchronize()
    return o.cpu().numpy(), (None if s is None else s.cpu().numpy())


def check(e, bs=None, hs=None, tol=WKV5_TOL):
    o, _ = gpu_finch(e)
    r, k, v, wt, u = (e[n] for n in ("r", "k", "v", "wt", "u"))
    if bs is not None:
        r, k, v, wt = r[bs], k[bs], v[bs], wt[bs]
        o = o[bs]
    if hs is not None:
        r, k, v, wt, u = r[:, :, hs], k[:, :, hs], v[:, :, hs], wt[:, :, hs], u[hs]
        o = o[:, :, hs]
    o_ref, _ = O.wkv6_recurrent(r, k, v, wt, u)
    o_abs, _ = O.wkv6_scale(r, k, v, wt, u)
    err = wkv5_scaled_err(o, o_ref, o_abs)
    log(f"  err={err:.3e}")
    assert err <= tol
    assert np.all(np.isfinite(o))
    return err


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 100, 3), (1, 257, 2), (3, 64, 1), (2, 200, 9)])
def test_small_shapes(shape):
    B, T, H = shape
    log(f"wkv6_forward B={B} T={T} H={H}")
    check(synth.wkv6_inputs(B, T, H, 64, seed=50 + T))


@pytest.mark.parametrize("case", [("fast", 2.0, 3.5, 0.5), ("mixed", -6.0, 3.0, 1.5),
                                  ("slow", -9.0, -6.0, 0.1)])
def test_decay_ranges(case):
    """fast: every |log2 w| > 15, every chunk computes its diagonal blocks
    exactly; mixed: chunks of both kinds; slow: decays very close to 1."""
    name, lo, hi, dstd = case
    log(f"wkv6_forward decays {name}")
    check(synth.wkv6_inputs(2, 300, 2, 64, seed=7, omega_lo=lo, omega_hi=hi, delta_std=dstd))


def test_extreme_decays():
    e = synth.wkv6_inputs(1, 200, 2, 64, seed=8)
    wt = e["wt"].copy()
    wt[:, 50:60] = 1e-30      # forget everything
    wt[:, 100:140] = 1.0      # remember everything
    log("wkv6_forward with w=1e-30 and w=1 stretches")
    check(dict(e, wt=wt))


def test_constant_decay_matches_eagle():
    torch, _ = torch_dev()
    e = synth.wkv6_inputs(2, 190, 3, 64, seed=9)
    wt = np.ascontiguousarray(np.broadcast_to(e["w"][None, None], e["wt"].shape))
    o6, _ = gpu_finch(dict(e, wt=wt))
    o5 = rw.rwkv_wkv5_forward(_bits(e, "r"), _bits(e, "k"), _bits(e, "v"), to_dev(e["w"]),
                              to_dev(e["u"]))
    torch.cuda.synchronize()
    o_abs = O.wkv5_scale(e["r"], e["k"], e["v"], e["w"], e["u"])
    o_ref, _ = O.wkv5_recurrent(e["r"], e["k"], e["v"], e["w"], e["u"])
    assert wkv5_scaled_err(o6, o_ref, o_abs) <= WKV5_TOL
    assert wkv5_scaled_err(o6, o5.cpu().numpy().astype(np.float64), o_abs) <= WKV5_TOL


def test_finch_workload_sampled_heads():
    cfg = synth.CFG_WKV6_FINCH
    log(f"wkv6_forward {cfg.name} (oracle on 2 batches x 3 heads)")
    e = synth.wkv6_inputs(cfg.B, cfg.T, cfg.H, cfg.D, cfg.seed)
    check(e, bs=np.array([0, 3]), hs=np.array([1, 16, 30]))


@pytest.mark.parametrize("cut", [(100, 5, 129), (128, 0, 64), (1, 2, 63)])
def test_forward_state_chain_matches_whole_sequence(cut):
    torch, dev = torch_dev()
    T1, N, T2 = cut
    B, H = 2, 3
    log(f"wkv6_forward/step chain {cut}")
    e = synth.wkv6_inputs(B, T1 + N + T2, H, 64, seed=70 + T1 + N, delta_std=1.0)
    u = to_dev(e["u"])
    sl = np.s_[:, :T1]
    o1, s = rw.rwkv_wkv6_forward(_bits(e, "r", sl), _bits(e, "k", sl), _bits(e, "v", sl),
                                 to_dev(e["wt"][sl]), u, s_out=True)
    outs = [o1]
    for t in range(T1, T1 + N):
        sl = np.s_[:, t]
        outs.append(rw.rwkv_wkv6_step(s, _bits(e, "r", sl), _bits(e, "k", sl), _bits(e, "v", sl),
                                      to_dev(e["wt"][sl]), u)[:, None])
    sl = np.s_[:, T1 + N:]
    o3, _ = rw.rwkv_wkv6_forward(_bits(e, "r", sl), _bits(e, "k", sl), _bits(e, "v", sl),
                                 to_dev(e["wt"][sl]), u, s_in=s, s_out=s)
    outs.append(o3)
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1).cpu().numpy()
    o_ref, s_ref = O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"])
    o_abs, s_abs = O.wkv6_scale(e["r"], e["k"], e["v"], e["wt"], e["u"])
    err_o = wkv5_scaled_err(o, o_ref, o_abs)
    err_s = wkv5_scaled_err(s.cpu().numpy(), s_ref, s_abs)
    log(f"  err o={err_o:.3e} state={err_s:.3e}")
    assert err_o <= WKV5_TOL and err_s <= WKV5_TOL


def test_steps_from_a_given_state():
    torch, dev = torch_dev()
    B, H, N = 3, 4, 30
    e = synth.wkv6_inputs(B, N, H, 64, seed=11, delta_std=1.0)
    s0 = np.random.default_rng(3).standard_normal((B, H, 64, 64)).astype(np.float32)
    s = to_dev(s0)
    outs = []
    for t in range(N):
        sl = np.s_[:, t]
        outs.append(rw.rwkv_wkv6_step(s, _bits(e, "r", sl), _bits(e, "k", sl), _bits(e, "v", sl),
                                      to_dev(e["wt"][sl]), to_dev(e["u"])))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=1).cpu().numpy()
    o_ref, s_ref = O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"], S0=s0)
    o_abs, s_abs = O.wkv6_scale(e["r"], e["k"], e["v"], e["wt"], e["u"], S0=s0)
    err_o = wkv5_scaled_err(o, o_ref, o_abs)
    err_s = wkv5_scaled_err(s.cpu().numpy(), s_ref, s_abs)
    log(f"  err o={err_o:.3e} state={err_s:.3e}")
    assert err_o <= 1e-5 and err_s <= 1e-5


@pytest.mark.parametrize("dv", ["64", "32"])
@pytest.mark.parametrize("segs", [1, 2, 3, 4])
def test_time_segments_and_slices(segs, dv):
    """Split over time segments (local end states and summed log-decays folded
    into later segments) and over value slices, with a starting state and the
    handed-on state; one chunk of fast decays takes the exact diagonal path."""
    torch, dev = torch_dev()
    e = synth.wkv6_inputs(2, 1000, 2, 64, seed=20 + segs, delta_std=1.0)
    wt = e["wt"].copy()
    wt[:, 300:340] = 1e-12
    e = dict(e, wt=wt)
    s0 = (np.random.default_rng(segs).standard_normal((2, 2, 64, 64)) * 0.3).astype(np.float32)
    log(f"wkv6_forward segments={segs} value columns={dv}")
    with tuned(wkv6_segs=segs, wkv6_dv=dv):
        o, s1 = gpu_finch(e, s_in=to_dev(s0), s_out=True)
    o_ref, s_ref = O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"], S0=s0)
    o_abs, s_abs = O.wkv6_scale(e["r"], e["k"], e["v"], e["wt"], e["u"], S0=s0)
    err_o = wkv5_scaled_err(o, o_ref, o_abs)
    err_s = wkv5_scaled_err(s1, s_ref, s_abs)
    log(f"  err o={err_o:.3e} state={err_s:.3e}")
    assert err_o <= WKV5_TOL and err_s <= WKV5_TOL


def test_query_factor_across_a_deep_block_decay():
    """A fast chunk whose second block starts with eight decays of 2^-14.9
    after sixteen of 2^-0.5: the total decay to that block's middle
    (2^-127.2) is below the float range, but the factor a query at the
    block's first token applies to the carried state, 2^-8, is not.  The
    factor must go through the block's first token (two ratios <= 1), not a
    ratio to the block middle that flushes to zero; a large starting state
    with small k, v makes the state term dominate the output."""
    torch, _ = torch_dev()
    B, T, H = 1, 64, 2
    log("wkv6_forward: deep decay at a block start, large carried state")
    e = synth.wkv6_inputs(B, T, H, 64, seed=77)
    wt = np.full((B, T, H, 64), 2.0 ** -0.5, np.float32)
    wt[:, 16:24] = np.float32(2.0 ** -14.9)
    small = {}
    for n in ("r", "k", "v"):
        x = e[n] if n == "r" else e[n] * np.float32(0.01)
        bits = synth.bf16_bits_from_f32(x)
        small[n], small[n + "_bits"] = synth.f32_from_bf16_bits(bits), bits
    e = dict(e, wt=wt, **small)
    s0 = (np.random.default_rng(3).standard_normal((B, H, 64, 64)) * 100).astype(np.float32)
    o, s1 = gpu_finch(e, s_in=to_dev(s0), s_out=True)
    o_ref, s_ref = O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"], S0=s0)
    o_abs, s_abs = O.wkv6_scale(e["r"], e["k"], e["v"], e["wt"], e["u"], S0=s0)
    err_o = wkv5_scaled_err(o, o_ref, o_abs)
    err_s = wkv5_scaled_err(s1, s_ref, s_abs)
    # the tokens whose factor would have flushed
    err_blk = wkv5_scaled_err(o[:, 16:24], o_ref[:, 16:24], o_abs[:, 16:24])
    log(f"  err o={err_o:.3e} (tokens 16..23: {err_blk:.3e}) state={err_s:.3e}")
    assert err_o <= WKV5_TOL and err_s <= WKV5_TOL

def test_most_heads_sampled():
    """H = 65535, the most the forward accepts (a chunk's rows of o span
    64 x H x 64 floats, 1.07 GB, under the 2^31-byte buffer range), T = 70
    (a ragged second chunk); six heads, the first and last included, against
    the oracle."""
    torch, dev = torch_dev()
    B, T, H, D = 1, 70, 65535, 64
    log(f"wkv6_forward B={B} T={T} H={H}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    r, k, v = ((torch.randn((B, T, H, D), generator=gen, device=dev) / 8).to(torch.bfloat16)
               for _ in range(3))
    omega = torch.rand((H, D), generator=gen, device=dev) * 6.0 - 6.0
    w = torch.exp(-torch.exp(omega))
    u = torch.randn((H, D), generator=gen, device=dev) * 0.5
    wt = torch.exp(-torch.exp(omega[None, None] + torch.randn((B, T, H, D), generator=gen,
                                                              device=dev) * 0.5))
    o, _ = rw.rwkv_wkv6_forward(r, k, v, wt, u)
    torch.cuda.synchronize()
    hs = torch.tensor([0, 1, 12345, 40000, H - 2, H - 1], device=dev)
    f = lambda x: x[:, :, hs].float().cpu().numpy()  # noqa: E731
    o_ref, _ = O.wkv6_recurrent(f(r), f(k), f(v), f(wt), u[hs].cpu().numpy())
    o_abs, _ = O.wkv6_scale(f(r), f(k), f(v), f(wt), u[hs].cpu().numpy())
    err = wkv5_scaled_err(f(o), o_ref, o_abs)
    log(f"  err={err:.3e} over {len(hs)} heads")
    assert err <= WKV5_TOL
    del r, k, v, o
    torch.cuda.empty_cache()
