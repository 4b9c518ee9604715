"""GPU parity of the RWKV-4 entry points against the fp64 oracle.

Tolerance (floating point): max |y_gpu - y_oracle| / S <= 1e-4, where S is
the oracle's weighted mean of |v| with the same weights (S >= |y|): the
condition scale of a convex combination.  Index-only properties (first
token, identity map, shift map) are checked bit for bit.
"""

import numpy as np
import pytest

import linear_attention_sequence_rwkv_amd as rw
import oracle.wkv_oracle as O
import synth
from wkv_testutil import WKV4_TOL, log, to_dev, torch_dev, tuned, wkv4_scaled_err

pytestmark = pytest.mark.gpu

TILE_VARIANTS = ["4,8,8", "4,16,4", "4,16,8", "2,16,8", "2,32,4", "2,16,4", "1,32,8",
                 "1,32,4", "1,64,1", "1,16,4", "1,32,4,2", "1,32,4,4"]


def _tile_settings(tile):
    return {"wkv4_tile": tile}


def gpu_forward(inp, tile=None):
    torch, _ = torch_dev()
    with tuned(**_tile_settings(tile)):
        y = rw.rwkv_wkv4_forward(to_dev(inp["w"]), to_dev(inp["u"]), to_dev(inp["k"]),
                                 to_dev(inp["v"]))
        torch.cuda.synchronize()
    return y.cpu().numpy()


def oracle_forward(inp, channels=None):
    w, u, k, v = inp["w"], inp["u"], inp["k"], inp["v"]
    if channels is not None:
        w, u, k, v = w[channels], u[channels], k[..., channels], v[..., channels]
    y, _ = O.wkv4_recurrent(w, u, k, v)
    S = O.wkv4_scale(w, u, k, v)
    return y, S


def test_tiny_workload_matches_direct_sum():
    cfg = synth.CFG_WKV4_TINY
    log(f"wkv4_forward {cfg.name} seed={cfg.seed}")
    inp = synth.wkv4_inputs_for(cfg)
    y = gpu_forward(inp)
    yd = O.wkv4_direct(inp["w"], inp["u"], inp["k"], inp["v"])
    S = O.wkv4_scale(inp["w"], inp["u"], inp["k"], inp["v"])
    err = wkv4_scaled_err(y, yd, S)
    log(f"  err={err:.3e}")
    assert err <= WKV4_TOL
    assert np.array_equal(y[:, 0, :], inp["v"][:, 0, :])


@pytest.mark.parametrize("tile", TILE_VARIANTS)
@pytest.mark.parametrize("shape", [(2, 1000, 200), (1, 777, 64), (3, 64, 65), (1, 1, 7),
                                   (2, 2051, 130)])
def test_ragged_shapes_all_tiles(shape, tile):
    B, T, C = shape
    log(f"wkv4_forward B={B} T={T} C={C} tile={tile}")
    inp = synth.wkv4_inputs(B, T, C, seed=17 + T + C, omega_lo=-5.0, omega_hi=2.0,
                            u_std=1.0, k_std=3.0)
    y = gpu_forward(inp, tile)
    y_ref, S = oracle_forward(inp)
    err = wkv4_scaled_err(y, y_ref, S)
    log(f"  err={err:.3e}")
    assert err <= WKV4_TOL
    assert np.array_equal(y[:, 0, :], inp["v"][:, 0, :])


def test_169m_width_workload_full():
    cfg = synth.CFG_WKV4_169M
    log(f"wkv4_forward {cfg.name} seed={cfg.seed}")
    inp = synth.wkv4_inputs_for(cfg)
    y = gpu_forward(inp)
    y_ref, S = oracle_forward(inp)
    err = wkv4_scaled_err(y, y_ref, S)
    log(f"  err={err:.3e}")
    assert err <= WKV4_TOL


def test_long_sequence_workload_sampled_channels():
    """B=1 T=65536 C=5120 on the GPU; the oracle runs 320 of the channels
    (every 16th, plus the last) over the full sequence."""
    cfg = synth.CFG_WKV4_LONG
    log(f"wkv4_forward {cfg.name} seed={cfg.seed} (oracle on sampled channels)")
    inp = synth.wkv4_inputs_for(cfg)
    y = gpu_forward(inp)
    ch = np.unique(np.concatenate([np.arange(0, cfg.C, 16), [cfg.C - 1]]))
    y_ref, S = oracle_forward(inp, ch)
    err = wkv4_scaled_err(y[..., ch], y_ref, S)
    log(f"  err={err:.3e} over {len(ch)} channels")
    assert err <= WKV4_TOL
    assert np.all(np.isfinite(y))


def test_identity_and_shift_maps_bit_exact():
    """u=+100: the current token dominates, y == v.  w=100, u=-100: only the
    previous token survives, y[t] == v[t-1].  Holds across tile boundaries."""
    B, T, C = 2, 1500, 192
    inp = synth.wkv4_inputs(B, T, C, seed=99)
    for tile in ("4,8,8", "2,16,4", "1,16,4"):
        log(f"wkv4_forward identity/shift maps tile={tile}")
        ident = dict(inp, u=np.full(C, 100.0, np.float32))
        assert np.array_equal(gpu_forward(ident, tile), inp["v"])
        shift = dict(inp, w=np.full(C, 100.0, np.float32), u=np.full(C, -100.0, np.float32))
        y = gpu_forward(shift, tile)
        assert np.array_equal(y[:, 0], inp["v"][:, 0])
        assert np.array_equal(y[:, 1:], inp["v"][:, :-1])


def test_identity_and_shift_maps_at_the_longest_sequence():
    """The longest sequence the forward accepts, T = 2^24 - 64 (its decay
    count is a float), with C = 128: 131,072 tiles per channel block, two
    blocks per workgroup, claimed tiles.  Both maps hold at any length, so
    the 8.6 GB outputs are checked whole, on the GPU: u = +100 gives y == v,
    w = 100 with u = -100 gives y[t] == v[t-1]."""
    torch, dev = torch_dev()
    B, T, C = 1, (1 << 24) - 64, 128
    log(f"wkv4_forward identity/shift maps at B={B} T={T} C={C}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    k = torch.randn((B, T, C), generator=gen, device=dev, dtype=torch.float32)
    v = torch.randn((B, T, C), generator=gen, device=dev, dtype=torch.float32)
    w = torch.rand((C,), generator=gen, device=dev, dtype=torch.float32) * 2.0
    y = torch.empty_like(k)
    rw.rwkv_wkv4_forward(w, torch.full((C,), 100.0, device=dev), k, v, y=y)
    torch.cuda.synchronize()
    assert torch.equal(y, v)
    rw.rwkv_wkv4_forward(torch.full((C,), 100.0, device=dev), torch.full((C,), -100.0, device=dev),
                         k, v, y=y)
    torch.cuda.synchronize()
    assert torch.equal(y[:, 0], v[:, 0])
    assert torch.equal(y[:, 1:], v[:, :-1])
    ws = rw.default_workspace("wkv4", dev)
    assert rw.rwkv_wkv4_workspace_error(ws) == 0
    del k, v, y
    torch.cuda.empty_cache()


def test_widest_rows_sampled_channels():
    """C = 2^22 + 37 channels (16 MB rows, a ragged last channel block): the
    row offsets within a wave's 32 rows and the channel-block indices are at
    their largest; 40 sampled channels, the last ones included, against the
    oracle."""
    torch, dev = torch_dev()
    B, T, C = 1, 200, (1 << 22) + 37
    log(f"wkv4_forward B={B} T={T} C={C}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(4321)
    k = torch.randn((B, T, C), generator=gen, device=dev, dtype=torch.float32)
    v = torch.randn((B, T, C), generator=gen, device=dev, dtype=torch.float32)
    w = torch.exp(torch.rand((C,), generator=gen, device=dev) * 4.0 - 3.0)
    u = torch.randn((C,), generator=gen, device=dev) * 0.5
    y = rw.rwkv_wkv4_forward(w, u, k, v)
    torch.cuda.synchronize()
    ch = np.concatenate([np.arange(0, C, C // 32), np.arange(C - 8, C)])
    cht = torch.from_numpy(ch).to(dev)
    inp = {"w": w[cht].cpu().numpy(), "u": u[cht].cpu().numpy(),
           "k": k[..., cht].cpu().numpy(), "v": v[..., cht].cpu().numpy()}
    y_ref, S = oracle_forward(inp)
    err = wkv4_scaled_err(y[..., cht].cpu().numpy(), y_ref, S)
    log(f"  err={err:.3e} over {len(ch)} channels")
    assert err <= WKV4_TOL
    del k, v, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("shift", [-80.0, 80.0])
def test_key_shift_stability(shift):
    B, T, C = 1, 3000, 128
    inp = synth.wkv4_inputs(B, T, C, seed=5, omega_lo=-5.0, omega_hi=2.0, u_std=1.0, k_std=3.0)
    log(f"wkv4_forward key shift {shift}")
    shifted = dict(inp, k=(inp["k"] + np.float32(shift)).astype(np.float32))
    y = gpu_forward(shifted)
    y_ref, S = oracle_forward(shifted)
    assert wkv4_scaled_err(y, y_ref, S) <= WKV4_TOL


def test_key_jumps_mix_blocked_and_exact_updates():
    """k ~ N(0, 15): in about half of the 8-token blocks some lane has a key
    ~100 log2 units above its history, and the wave takes the exact per-token
    update there; the other blocks take the one-exp2 update, so the history
    passes between the two forms many times per sequence."""
    B, T, C = 2, 3000, 256
    inp = synth.wkv4_inputs(B, T, C, seed=8, omega_lo=-5.0, omega_hi=2.0, u_std=1.0,
                            k_std=15.0)
    log("wkv4_forward key jumps k_std=15")
    y = gpu_forward(inp)
    y_ref, S = oracle_forward(inp)
    assert wkv4_scaled_err(y, y_ref, S) <= WKV4_TOL


def test_zero_decay_long_average():
    B, T, C = 1, 20000, 64
    inp = synth.wkv4_inputs(B, T, C, seed=6)
    inp["w"] = np.zeros(C, np.float32)
    log("wkv4_forward w=0")
    y = gpu_forward(inp)
    y_ref, S = oracle_forward(inp)
    assert wkv4_scaled_err(y, y_ref, S) <= WKV4_TOL


def test_workspace_reuse_across_shapes():
    """The cached workspace keeps working across many calls and shapes."""
    a = synth.wkv4_inputs(2, 900, 96, seed=1)
    b = synth.wkv4_inputs(1, 5000, 300, seed=2)
    ya_ref, Sa = oracle_forward(a)
    yb_ref, Sb = oracle_forward(b)
    log("wkv4_forward 40 alternating calls")
    for i in range(20):
        assert wkv4_scaled_err(gpu_forward(a), ya_ref, Sa) <= WKV4_TOL, i
        assert wkv4_scaled_err(gpu_forward(b), yb_ref, Sb) <= WKV4_TOL, i


def test_in_order_and_claimed_launches_share_a_workspace():
    """A grid the device holds at once takes tiles in launch order; a larger
    one (here 32 tiles x 96 channel blocks) claims them in arrival order.
    Both advance the same workspace epoch: alternate them on one workspace."""
    torch, dev = torch_dev()
    shapes = [(2, 900, 96), (4, 4096, 1536)]
    cases = [synth.wkv4_inputs(B, T, C, seed=90 + i) for i, (B, T, C) in enumerate(shapes)]
    refs = [oracle_forward(inp) for inp in cases]
    need = max(rw.rwkv_wkv4_forward_workspace(*shp) for shp in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    bufs = [{n: to_dev(inp[n]) for n in ("w", "u", "k", "v")} for inp in cases]
    for rnd in range(3):
        for shp, bf, (y_ref, S) in zip(shapes, bufs, refs):
            log(f"wkv4_forward shared workspace round {rnd} shape {shp}")
            y = rw.rwkv_wkv4_forward(bf["w"], bf["u"], bf["k"], bf["v"], ws=ws)
            torch.cuda.synchronize()
            assert wkv4_scaled_err(y.cpu().numpy(), y_ref, S) <= WKV4_TOL, (rnd, shp)


@pytest.mark.parametrize("cfg_name", ["169m", "tiny", "ragged"])
def test_launch_order_and_claimed_tiles_give_the_same_bits(cfg_name):
    """Tiles taken in launch order (the whole grid resident) and claimed in
    arrival order fold the same histories in the same chain order: the
    outputs and the final state must agree bit for bit
    (the RWKV_TUNE_WKV4_ORDER override forces claims)."""
    torch, dev = torch_dev()
    if cfg_name == "ragged":
        inp = synth.wkv4_inputs(3, 1100, 200, seed=77)
    else:
        cfg = synth.CFG_WKV4_169M if cfg_name == "169m" else synth.CFG_WKV4_TINY
        inp = synth.wkv4_inputs_for(cfg)
    B, T, C = inp["k"].shape
    g = np.random.default_rng(5)
    st = [torch.from_numpy(x.astype(np.float32)).to(dev)
          for x in (g.random((B, C)), g.random((B, C)) + 0.5, g.normal(size=(B, C)))]
    t = {n: torch.from_numpy(inp[n]).to(dev) for n in ("w", "u", "k", "v")}
    outs = {}
    for mode in ("", "claim"):
        log(f"wkv4_forward {B}x{T}x{C}: prefix mode {mode or 'default'}, bitwise")
        with tuned(wkv4_claim=mode == "claim"):
            y = rw.rwkv_wkv4_forward(t["w"], t["u"], t["k"], t["v"])
            y2, (a2, b2, p2) = rw.rwkv_wkv4_forward_state(t["w"], t["u"], t["k"], t["v"],
                                                         state_in=tuple(st), state_out=True)
            torch.cuda.synchronize()
        outs[mode] = [x.cpu().numpy() for x in (y, y2, a2, b2, p2)]
    for x, z in zip(outs[""], outs["claim"]):
        assert np.array_equal(x, z)


def test_concurrent_streams_with_launch_order():
    """Two 8x1024x768 forwards on two streams at once, each grid resident on
    its own but not both together: a tile still only waits on workgroups
    dispatched before it.  Both results must match the oracle."""
    torch, dev = torch_dev()
    cfg = synth.CFG_WKV4_169M
    inps = [synth.wkv4_inputs(cfg.B, cfg.T, cfg.C, seed=140 + i) for i in range(2)]
    refs = [oracle_forward(inp) for inp in inps]
    need = rw.rwkv_wkv4_forward_workspace(cfg.B, cfg.T, cfg.C)
    streams = [torch.cuda.Stream(dev) for _ in range(2)]
    bufs, wss, ys = [], [], []
    for inp in inps:
        bufs.append({n: to_dev(inp[n]) for n in ("w", "u", "k", "v")})
        wss.append(torch.zeros(need, dtype=torch.uint8, device=dev))
        ys.append(torch.empty_like(bufs[-1]["k"]))
    torch.cuda.synchronize()
    for rnd in range(3):
        log(f"wkv4_forward two streams round {rnd}")
        for st, bf, ws, y in zip(streams, bufs, wss, ys):
            with torch.cuda.stream(st):
                rw.rwkv_wkv4_forward(bf["w"], bf["u"], bf["k"], bf["v"], y=y, ws=ws)
        torch.cuda.synchronize()
        for y, (y_ref, S) in zip(ys, refs):
            assert wkv4_scaled_err(y.cpu().numpy(), y_ref, S) <= WKV4_TOL, rnd


def test_workspace_layout_changes():
    """Regression: one workspace serves calls whose channel-block counts grow
    and shrink, so earlier calls' words sit where later calls keep their
    counters and histories."""
    shapes = [(1, 300, 64), (4, 300, 771), (1, 700, 5120), (8, 300, 770), (2, 300, 64),
              (16, 200, 1028)]
    cases = [(synth.wkv4_inputs(B, T, C, seed=3 + i), (B, T, C)) for i, (B, T, C) in enumerate(shapes)]
    refs = [oracle_forward(inp) for inp, _ in cases]
    for rnd in range(2):
        for (inp, shp), (y_ref, S) in zip(cases, refs):
            log(f"wkv4_forward layout change round {rnd} shape {shp}")
            assert wkv4_scaled_err(gpu_forward(inp), y_ref, S) <= WKV4_TOL, shp


def test_forward_replayed_from_captured_graph():
    """Calls captured in a HIP graph and replayed must still see fresh
    workspace tags: replay several times, with eager calls on the same
    workspace and new inputs in between, and check every replay."""
    torch, dev = torch_dev()
    shapes = [(2, 900, 96), (1, 1500, 320)]
    inps = [synth.wkv4_inputs(B, T, C, seed=60 + i) for i, (B, T, C) in enumerate(shapes)]
    alts = [synth.wkv4_inputs(B, T, C, seed=70 + i) for i, (B, T, C) in enumerate(shapes)]
    need = max(rw.rwkv_wkv4_forward_workspace(*shp) for shp in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    bufs = [{n: to_dev(inp[n]) for n in ("w", "u", "k", "v")} for inp in inps]
    ys = [torch.empty_like(bf["k"]) for bf in bufs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(graph, stream=side):
        for bf, y in zip(bufs, ys):
            rw.rwkv_wkv4_forward(bf["w"], bf["u"], bf["k"], bf["v"], y=y, ws=ws)
    torch.cuda.synchronize()
    for rnd in range(4):
        src = inps if rnd % 2 == 0 else alts
        for bf, inp in zip(bufs, src):
            for n in ("w", "u", "k", "v"):
                bf[n].copy_(to_dev(inp[n]))
        # eager calls on the same workspace between replays
        for bf, y in zip(bufs, ys):
            rw.rwkv_wkv4_forward(bf["w"], bf["u"], bf["k"], bf["v"], ws=ws)
        torch.cuda.synchronize()
        log(f"wkv4_forward graph replay {rnd}")
        graph.replay()
        torch.cuda.synchronize()
        for y, inp in zip(ys, src):
            y_ref, S = oracle_forward(inp)
            assert wkv4_scaled_err(y.cpu().numpy(), y_ref, S) <= WKV4_TOL, rnd


# ------------------------------------------------------------------ step ---

def _run_steps(inp, n_steps, pool=None):
    torch, dev = torch_dev()
    B, C = inp["k"].shape[-2:]
    w, u = to_dev(inp["w"]), to_dev(inp["u"])
    k_all, v_all = to_dev(inp["k"]), to_dev(inp["v"])
    a, b, p = rw.rwkv_wkv4_state_init(B, C, device=dev)
    ys = []
    for t in range(n_steps):
        i = t % pool if pool else t
        ys.append(rw.rwkv_wkv4_step(a, b, p, w, u, k_all[i], v_all[i]))
    torch.cuda.synchronize()
    return torch.stack(ys).cpu().numpy(), (a.cpu().numpy(), b.cpu().numpy(), p.cpu().numpy())


@pytest.mark.parametrize("C", [768, 771])
def test_steps_match_oracle_and_forward(C):
    B, N = 4, 300
    fwd = synth.wkv4_inputs(B, N, C, seed=31)
    log(f"wkv4_step B={B} C={C} x{N}")
    step_inp = dict(fwd, k=np.ascontiguousarray(fwd["k"].transpose(1, 0, 2)),
                    v=np.ascontiguousarray(fwd["v"].transpose(1, 0, 2)))
    ys, (a, b, p) = _run_steps(step_inp, N)
    ys = ys.transpose(1, 0, 2)  # -> [B, N, C]
    y_ref, st = O.wkv4_recurrent(fwd["w"], fwd["u"], fwd["k"], fwd["v"])
    S = O.wkv4_scale(fwd["w"], fwd["u"], fwd["k"], fwd["v"])
    assert wkv4_scaled_err(ys, y_ref, S) <= WKV4_TOL
    assert np.array_equal(ys[:, 0], fwd["v"][:, 0])
    # step mode and the time-parallel forward agree
    y_fwd = gpu_forward(fwd)
    assert wkv4_scaled_err(ys, y_fwd.astype(np.float64), S) <= 2 * WKV4_TOL
    # state: only a/b and log(b)+p are defined
    mean_ref, logden_ref = O.wkv4_canonical_state(st)
    a64, b64, p64 = (x.astype(np.float64) for x in (a, b, p))
    Sv = np.abs(fwd["v"]).max(axis=1)
    assert np.max(np.abs(a64 / b64 - mean_ref) / Sv) <= WKV4_TOL
    assert np.max(np.abs(np.log(b64) + p64 - logden_ref)) <= 1e-4 * (1 + np.abs(logden_ref)).max()


def test_state_init_is_empty():
    torch, dev = torch_dev()
    a, b, p = rw.rwkv_wkv4_state_init(3, 70, device=dev)
    torch.cuda.synchronize()
    assert torch.all(a == 0) and torch.all(b == 0)
    assert torch.all(p == torch.tensor(-1e38, dtype=torch.float32, device=dev))


def test_decode_workload_sampled_lanes():
    """B=256 C=4096, 4096 steps from a pool of 64 token draws; the oracle
    follows 512 sampled (stream, channel) lanes through all steps."""
    torch, dev = torch_dev()
    cfg = synth.CFG_WKV4_DECODE
    log(f"wkv4_step {cfg.name} seed={cfg.seed}")
    inp = synth.wkv4_step_inputs(cfg.B, cfg.C, cfg.pool, cfg.seed)
    rng = np.random.default_rng(0)
    lanes = np.sort(rng.choice(cfg.B * cfg.C, size=512, replace=False))
    lanes_t = torch.from_numpy(lanes).to(dev)
    w, u = to_dev(inp["w"]), to_dev(inp["u"])
    k_all, v_all = to_dev(inp["k"]), to_dev(inp["v"])
    a, b, p = rw.rwkv_wkv4_state_init(cfg.B, cfg.C, device=dev)
    y = torch.empty((cfg.B, cfg.C), dtype=torch.float32, device=dev)
    got = torch.empty((cfg.steps, len(lanes)), dtype=torch.float32, device=dev)
    for t in range(cfg.steps):
        i = t % cfg.pool
        rw.rwkv_wkv4_step(a, b, p, w, u, k_all[i], v_all[i], y=y)
        got[t] = y.view(-1)[lanes_t]
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    bi, ci = lanes // cfg.C, lanes % cfg.C
    kk = inp["k"][:, bi, ci]          # [pool, L]
    vv = inp["v"][:, bi, ci]
    idx = np.arange(cfg.steps) % cfg.pool
    k_seq = kk[idx][None]             # [1, steps, L]
    v_seq = vv[idx][None]
    y_ref, _ = O.wkv4_recurrent(inp["w"][ci], inp["u"][ci], k_seq, v_seq)
    S = O.wkv4_scale(inp["w"][ci], inp["u"][ci], k_seq, v_seq)
    err = wkv4_scaled_err(got[None], y_ref, S)
    log(f"  err={err:.3e}")
    assert err <= WKV4_TOL


# ------------------------------------------------- forward with a state ---

def _with_tile(tile, fn):
    with tuned(**_tile_settings(tile)):
        return fn()


@pytest.mark.parametrize("tile", [None, "4,8,8", "2,16,4", "1,64,1", "1,32,4,2"])
@pytest.mark.parametrize("cut", [(500, 7, 333), (40, 0, 1), (1, 3, 1000), (256, 1, 64)])
def test_forward_state_chain_matches_whole_sequence(cut, tile):
    """forward(T1) -> N steps -> forward(T2), the state handed on each time
    (the last hand-over in place), equals one pass over T1+N+T2 tokens."""
    torch, dev = torch_dev()
    T1, N, T2 = cut
    B, C = 3, 200
    log(f"wkv4_forward_state B={B} C={C} cut={cut} tile={tile}")
    inp = synth.wkv4_inputs(B, T1 + N + T2, C, seed=90 + T1 + T2)
    w, u = to_dev(inp["w"]), to_dev(inp["u"])
    k, v = to_dev(inp["k"]), to_dev(inp["v"])

    def run():
        y1, st = rw.rwkv_wkv4_forward_state(w, u, k[:, :T1].contiguous(),
                                            v[:, :T1].contiguous(), state_out=True)
        ys = [y1]
        for t in range(T1, T1 + N):
            ys.append(rw.rwkv_wkv4_step(*st, w, u, k[:, t].contiguous(),
                                        v[:, t].contiguous())[:, None])
        y3, _ = rw.rwkv_wkv4_forward_state(w, u, k[:, T1 + N:].contiguous(),
                                           v[:, T1 + N:].contiguous(), state_in=st,
                                           state_out=st)
        ys.append(y3)
        torch.cuda.synchronize()
        return torch.cat(ys, dim=1).cpu().numpy(), [x.cpu().numpy() for x in st]

    y, (a, b, p) = _with_tile(tile, run)
    y_ref, st_ref = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
    S = O.wkv4_scale(inp["w"], inp["u"], inp["k"], inp["v"])
    err = wkv4_scaled_err(y, y_ref, S)
    log(f"  err={err:.3e}")
    assert err <= WKV4_TOL
    mean_ref, logden_ref = O.wkv4_canonical_state(st_ref)
    a64, b64, p64 = (x.astype(np.float64) for x in (a, b, p))
    Sv = np.abs(inp["v"]).max(axis=1)
    assert np.max(np.abs(a64 / b64 - mean_ref) / Sv) <= WKV4_TOL
    assert np.max(np.abs(np.log(b64) + p64 - logden_ref)) <= 1e-4 * (1 + np.abs(logden_ref)).max()


def test_forward_state_without_states_is_the_plain_forward():
    torch, dev = torch_dev()
    inp = synth.wkv4_inputs(2, 700, 130, seed=5)
    y0 = gpu_forward(inp)
    y1, st = rw.rwkv_wkv4_forward_state(to_dev(inp["w"]), to_dev(inp["u"]), to_dev(inp["k"]),
                                        to_dev(inp["v"]))
    torch.cuda.synchronize()
    assert st is None
    assert np.array_equal(y0, y1.cpu().numpy())


def test_forward_state_from_empty_state_init():
    """An explicit empty state (state_init) gives the plain forward's output."""
    torch, dev = torch_dev()
    B, T, C = 2, 300, 96
    inp = synth.wkv4_inputs(B, T, C, seed=6)
    st = rw.rwkv_wkv4_state_init(B, C, device=dev)
    y, _ = rw.rwkv_wkv4_forward_state(to_dev(inp["w"]), to_dev(inp["u"]), to_dev(inp["k"]),
                                      to_dev(inp["v"]), state_in=st)
    torch.cuda.synchronize()
    y_ref, S = oracle_forward(inp)
    assert wkv4_scaled_err(y.cpu().numpy(), y_ref, S) <= WKV4_TOL


@pytest.mark.parametrize("cfg_name", ["169m", "long"])
def test_forward_is_deterministic(cfg_name):
    """Repeated calls give the same bits: the look-back folds predecessors in
    chain order whatever the timing (the long workload has 512 tiles per
    channel block, so deep look-backs do happen)."""
    torch, dev = torch_dev()
    cfg = synth.CFG_WKV4_169M if cfg_name == "169m" else synth.CFG_WKV4_LONG
    log(f"wkv4_forward {cfg.name} x3 bitwise")
    inp = synth.wkv4_inputs_for(cfg)
    w, u, k, v = (to_dev(inp[n]) for n in ("w", "u", "k", "v"))
    y0 = rw.rwkv_wkv4_forward(w, u, k, v)
    for _ in range(2):
        y1 = rw.rwkv_wkv4_forward(w, u, k, v)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)


@pytest.mark.parametrize("shape", [(8, 1024, 768), (3, 1100, 256), (1, 65536, 5120)])
def test_channel_block_groups_give_the_same_bits(shape):
    """Workgroups of 2 or 4 adjacent channel blocks keep every block's own
    128-token tiles, histories and look-back: outputs and final states equal
    those of one block per workgroup bit for bit, in launch order and with
    claimed tiles, on one shared workspace."""
    torch, dev = torch_dev()
    B, T, C = shape
    inp = synth.wkv4_inputs(B, T, C, seed=51 + T, omega_lo=-5.0, omega_hi=2.0, u_std=1.0,
                            k_std=3.0)
    g = np.random.default_rng(9)
    st = [torch.from_numpy(x.astype(np.float32)).to(dev)
          for x in (g.random((B, C)), g.random((B, C)) + 0.5, g.normal(size=(B, C)))]
    t = {n: torch.from_numpy(inp[n]).to(dev) for n in ("w", "u", "k", "v")}
    ws = torch.zeros(rw.rwkv_wkv4_forward_workspace(B, T, C), dtype=torch.uint8, device=dev)
    outs = {}
    for tile in ("1,32,4", "1,32,4,2", "1,32,4,4"):
        for claim in (False, True):
            log(f"wkv4_forward {B}x{T}x{C} tile {tile} claim={claim}, bitwise")
            with tuned(wkv4_tile=tile, wkv4_claim=claim):
                y = rw.rwkv_wkv4_forward(t["w"], t["u"], t["k"], t["v"], ws=ws)
                y2, (a2, b2, p2) = rw.rwkv_wkv4_forward_state(
                    t["w"], t["u"], t["k"], t["v"], state_in=tuple(st), state_out=True, ws=ws)
                torch.cuda.synchronize()
            outs[(tile, claim)] = [x.cpu().numpy() for x in (y, y2, a2, b2, p2)]
    ref = outs[("1,32,4", False)]
    for key, got in outs.items():
        for i, (x, z) in enumerate(zip(ref, got)):
            assert np.array_equal(x, z), (key, i)
    assert rw.rwkv_wkv4_workspace_error(ws) == 0
