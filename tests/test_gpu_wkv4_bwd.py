"""GPU parity of the RWKV-4 backward against the fp64 oracle.

Tolerance: for each gradient, max |g_gpu - g_oracle| / g_abs <= 1e-4, where
g_abs is the same sum with every term replaced by its magnitude bound
(oracle.wkv4_backward_scale): float32 rounding of a sum is relative to the
sum of its terms' magnitudes, not to the (possibly cancelling) result.
"""
import numpy as np
import pytest

import linear_attention_sequence_rwkv_amd as rw
import oracle.wkv_oracle as O
import synth
from wkv_testutil import WKV4_TOL, log, to_dev, torch_dev, tuned, wkv4_scaled_err

pytestmark = pytest.mark.gpu

NAMES = ("gw", "gu", "gk", "gv")


def gpu_backward(inp):
    torch, _ = torch_dev()
    out = rw.rwkv_wkv4_backward(to_dev(inp["w"]), to_dev(inp["u"]), to_dev(inp["k"]),
                                to_dev(inp["v"]), to_dev(inp["gy"]))
    torch.cuda.synchronize()
    return [o.cpu().numpy().astype(np.float64) for o in out]


def errors(got, ref, scale):
    return {n: float(np.max(np.abs(g - r) / np.maximum(s, 1e-30))) if g.size else 0.0
            for n, g, r, s in zip(NAMES, got, ref, scale)}


def check(inp, channels=None, tol=WKV4_TOL):
    got = gpu_backward(inp)
    w, u, k, v, gy = (inp[n] for n in ("w", "u", "k", "v", "gy"))
    if channels is not None:
        w, u, k, v, gy = w[channels], u[channels], k[..., channels], v[..., channels], \
            gy[..., channels]
        got = [g[..., channels] for g in got]
    ref = O.wkv4_backward_recurrent(w, u, k, v, gy)
    scale = O.wkv4_backward_scale(w, u, k, v, gy)
    err = errors(got, ref, scale)
    log("  " + " ".join(f"{n}={e:.2e}" for n, e in err.items()))
    for n, e in err.items():
        assert e <= tol, (n, e)
    for g in got:
        assert np.all(np.isfinite(g))


def test_tiny_workload_matches_the_definition():
    inp = synth.wkv4_backward_inputs(1, 64, 64, 1001)
    log("wkv4_backward B=1 T=64 C=64 vs direct definition")
    got = gpu_backward(inp)
    ref = O.wkv4_backward_direct(*(inp[n] for n in ("w", "u", "k", "v", "gy")))
    scale = O.wkv4_backward_scale(*(inp[n] for n in ("w", "u", "k", "v", "gy")))
    err = errors(got, ref, scale)
    log("  " + " ".join(f"{n}={e:.2e}" for n, e in err.items()))
    assert max(err.values()) <= WKV4_TOL


@pytest.mark.parametrize("shape", [(2, 1000, 200), (1, 777, 64), (3, 64, 65), (1, 1, 7),
                                   (2, 65, 130), (1, 17, 3), (2, 129, 64)])
def test_ragged_shapes(shape):
    B, T, C = shape
    log(f"wkv4_backward B={B} T={T} C={C}")
    check(synth.wkv4_backward_inputs(B, T, C, seed=3 + T + C))


def test_169m_width_workload_full():
    cfg = synth.CFG_WKV4_169M
    log(f"wkv4_backward {cfg.name} (full oracle)")
    check(synth.wkv4_backward_inputs(cfg.B, cfg.T, cfg.C, cfg.seed))


def test_long_sequence_workload_sampled_channels():
    cfg = synth.CFG_WKV4_LONG
    log(f"wkv4_backward {cfg.name} (oracle on 40 sampled channels)")
    inp = synth.wkv4_backward_inputs(cfg.B, cfg.T, cfg.C, cfg.seed, omega_lo=cfg.omega_lo,
                                     omega_hi=cfg.omega_hi, u_std=cfg.u_std, k_std=cfg.k_std)
    chans = np.sort(np.random.default_rng(2).choice(cfg.C, 40, replace=False))
    check(inp, channels=chans)


@pytest.mark.parametrize("shift", [-80.0, 80.0])
def test_key_shift_stability(shift):
    inp = synth.wkv4_backward_inputs(2, 500, 96, seed=21)
    inp = dict(inp, k=(inp["k"].astype(np.float64) + shift).astype(np.float32))
    log(f"wkv4_backward k{shift:+.0f}")
    check(inp)


def test_backward_is_deterministic():
    torch, _ = torch_dev()
    cfg = synth.CFG_WKV4_169M
    inp = synth.wkv4_backward_inputs(cfg.B, cfg.T, cfg.C, cfg.seed)
    args = [to_dev(inp[n]) for n in ("w", "u", "k", "v", "gy")]
    first = rw.rwkv_wkv4_backward(*args)
    for _ in range(2):
        again = rw.rwkv_wkv4_backward(*args)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)


@pytest.mark.parametrize("shape", [(8, 1024, 768), (3, 1100, 200)])
def test_launch_order_and_claimed_tiles_give_the_same_gradients(shape):
    """The prefix pass takes its tiles in launch order when the grid fits on
    the device and claims them otherwise (RWKV_WKV4_ORDER=claim forces
    claims); the folds run in the same chain order, so all four gradients
    must agree bit for bit, also when the two modes alternate on one
    workspace."""
    torch, _ = torch_dev()
    B, T, C = shape
    inp = synth.wkv4_backward_inputs(B, T, C, seed=91)
    args = [to_dev(inp[n]) for n in ("w", "u", "k", "v", "gy")]
    ws = torch.zeros(max(rw.rwkv_wkv4_backward_workspace(B, T, C), 256), dtype=torch.uint8,
                     device=args[0].device)
    outs = {}
    for rnd in range(2):
        for mode in ("", "claim"):
            log(f"wkv4_backward {shape}: tile order {mode or 'default'} round {rnd}")
            with tuned(wkv4_claim=mode == "claim"):
                got = rw.rwkv_wkv4_backward(*args, ws=ws)
                torch.cuda.synchronize()
            got = [x.cpu() for x in got]
            if mode in outs:
                for a, b in zip(outs[mode], got):
                    assert torch.equal(a, b), (mode, rnd)
            outs[mode] = got
    for a, b in zip(outs[""], outs["claim"]):
        assert torch.equal(a, b)


def test_backward_after_forward_calls_of_other_shapes():
    """The two workspaces (forward's, backward's) are independent; calls of
    different shapes in any order stay correct."""
    torch, _ = torch_dev()
    for B, T, C in ((1, 300, 64), (2, 70, 130), (1, 300, 64)):
        inp = synth.wkv4_backward_inputs(B, T, C, seed=B + T + C)
        rw.rwkv_wkv4_forward(to_dev(inp["w"]), to_dev(inp["u"]), to_dev(inp["k"]),
                             to_dev(inp["v"]))
        check(inp)


def test_workspace_layout_changes():
    """One cached workspace through calls whose layouts differ (large to
    small and back): wherever a call's counters land, the words it finds
    there carry earlier tags, so every call claims all of its tiles."""
    for B, T, C in ((1, 4096, 256), (1, 300, 64), (3, 64, 65), (2, 1000, 200), (1, 300, 64),
                    (4, 2048, 64)):
        log(f"wkv4_backward B={B} T={T} C={C} (shared workspace)")
        check(synth.wkv4_backward_inputs(B, T, C, seed=T + C))


def test_claimed_and_in_order_prefix_passes_share_a_workspace():
    """The prefix pass takes its tiles in launch order when its grid is
    resident at once (then primes the reverse pass's counters itself) and
    claims them otherwise (1 x 16384 x 4096: 8192 tiles); alternate the two
    on the cached workspace."""
    big = synth.wkv4_backward_inputs(1, 16384, 4096, seed=11)
    small = synth.wkv4_backward_inputs(2, 1000, 200, seed=12)
    ch = np.arange(0, 4096, 128)
    for rnd in range(2):
        log(f"wkv4_backward claimed prefix pass round {rnd} (sampled channels)")
        check(big, ch)
        log(f"wkv4_backward in-order prefix pass round {rnd}")
        check(small)


@pytest.mark.parametrize("shape", [(8, 1024, 768), (3, 1100, 200), (2, 300, 96), (1, 64, 64),
                                   (1, 16384, 256), (1, 65536, 1024)])
def test_training_pair_matches_the_separate_calls(shape):
    """rwkv_wkv4_forward_train leaves the prefix pass's tile histories in a
    backward workspace and rwkv_wkv4_backward_after_forward reuses them: y is
    within the bound of the oracle (and equal to rwkv_wkv4_forward's where both
    use the same tiles), and the gradients equal rwkv_wkv4_backward's bit for
    bit; a pair of another shape on another workspace in between changes
    nothing.  The last shape (8192 tiles of 128 x 64) runs the prefix pass and
    the training forward with two channel blocks per workgroup."""
    torch, dev = torch_dev()
    B, T, C = shape
    inp = synth.wkv4_backward_inputs(B, T, C, seed=303)
    args = [to_dev(inp[n]) for n in ("w", "u", "k", "v")]
    gy = to_dev(inp["gy"])
    need = rw.rwkv_wkv4_backward_workspace(B, T, C)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    other = synth.wkv4_backward_inputs(2, 700, 128, seed=304)
    oargs = [to_dev(other[n]) for n in ("w", "u", "k", "v", "gy")]
    ows = torch.zeros(max(rw.rwkv_wkv4_backward_workspace(2, 700, 128), 256),
                      dtype=torch.uint8, device=dev)
    ref_grads = [x.cpu() for x in rw.rwkv_wkv4_backward(*args, gy)]
    y_plain = rw.rwkv_wkv4_forward(*args).cpu().numpy()
    if T <= 4096:
        y_ref, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
        S = O.wkv4_scale(inp["w"], inp["u"], inp["k"], inp["v"])
    for rnd in range(2):
        log(f"wkv4 training pair {shape} round {rnd}")
        y = rw.rwkv_wkv4_forward_train(*args, ws=ws)
        if rnd == 1:
            rw.rwkv_wkv4_forward_train(*oargs[:4], ws=ows)
            rw.rwkv_wkv4_backward_after_forward(*oargs, ws=ows)
        grads = rw.rwkv_wkv4_backward_after_forward(*args, gy, ws=ws)
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        if T <= 4096:
            assert wkv4_scaled_err(y, y_ref, S) <= WKV4_TOL
        if T > 64:  # both calls tile 128 tokens with one channel per lane
            assert np.array_equal(y, y_plain)
        for a, b in zip(ref_grads, grads):
            assert torch.equal(a, b.cpu())


def test_identity_map_gradients_at_the_longest_sequence():
    """The backward at the longest sequence the forward accepts (T = 2^24 - 64,
    C = 128: 262,144 reverse tiles per block).  With u = +100 every output is
    its own token's v (p_tt = 1, every other weight below e^-90), so
    gv = gy and gk, gw, gu vanish; checked over the whole 8.6 GB gradients on
    the GPU."""
    torch, dev = torch_dev()
    B, T, C = 1, (1 << 24) - 64, 128
    log(f"wkv4_backward identity map at B={B} T={T} C={C}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(2468)
    k = torch.randn((B, T, C), generator=gen, device=dev, dtype=torch.float32)
    v = torch.randn((B, T, C), generator=gen, device=dev, dtype=torch.float32)
    gy = torch.randn((B, T, C), generator=gen, device=dev, dtype=torch.float32)
    w = torch.rand((C,), generator=gen, device=dev, dtype=torch.float32) * 2.0
    u = torch.full((C,), 100.0, device=dev)
    gw, gu, gk, gv = rw.rwkv_wkv4_backward(w, u, k, v, gy)
    torch.cuda.synchronize()
    rel = ((gv - gy).abs() / gy.abs().clamp_min(1e-30)).max().item()
    log(f"  max |gv - gy| / |gy| = {rel:.2e}, max |gk| = {gk.abs().max().item():.2e}, "
        f"max |gw| = {gw.abs().max().item():.2e}, max |gu| = {gu.abs().max().item():.2e}")
    assert rel <= 1e-6
    assert gk.abs().max().item() <= 1e-5
    assert gw.abs().max().item() <= 1e-4 and gu.abs().max().item() <= 1e-4
    ws = rw.default_workspace("wkv4_bwd", dev)
    assert rw.rwkv_wkv4_workspace_error(ws) == 0
    del k, v, gy, gk, gv
    torch.cuda.empty_cache()
