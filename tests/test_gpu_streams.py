"""Every entry point of the binding called on a stream other than torch's
current one (``stream=side``): the outputs and workspaces the binding
allocates are allocated and zero-filled on that stream, ahead of the call,
so the results equal, bit for bit, those of the same call on the current
stream (every kernel here is deterministic).  The side stream first waits
for the current one (the inputs are made there), and the current stream
waits for the side one before the results are read, as torch's stream
semantics ask of any caller.  Each call runs twice on the side stream, so
the side stream's cached workspace is reused once."""
import numpy as np
import pytest

import linear_attention_sequence_rwkv_amd as rw
import synth
from wkv_testutil import log, to_dev, torch_dev

pytestmark = pytest.mark.gpu


def _side(torch, dev):
    side = torch.cuda.Stream(dev)  # default priority
    side.wait_stream(torch.cuda.current_stream(dev))
    return side


def _same(torch, dev, side, ref, got, what):
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ref, got)):
        if a is None:
            assert b is None
            continue
        assert torch.equal(a, b), f"{what}: output {i} differs on the side stream"


def _wkv4(torch):
    e = synth.wkv4_backward_inputs(2, 300, 200, seed=31)
    return {n: to_dev(e[n]) for n in ("w", "u", "k", "v", "gy")}


def test_wkv4_forward_entry_points_on_a_side_stream():
    torch, dev = torch_dev()
    t = _wkv4(torch)
    args = (t["w"], t["u"], t["k"], t["v"])
    ref_y = rw.rwkv_wkv4_forward(*args)
    ref_s = rw.rwkv_wkv4_forward_state(*args, state_out=True)
    ref_n = rw.rwkv_wkv4_forward_noalloc(*args)
    side = _side(torch, dev)
    for rep in range(2):
        log(f"wkv4 forward entry points on a side stream, call {rep}")
        y = rw.rwkv_wkv4_forward(*args, stream=side)
        ys, (a, b, p) = rw.rwkv_wkv4_forward_state(*args, state_out=True, stream=side)
        yn = rw.rwkv_wkv4_forward_noalloc(*args, stream=side)
        _same(torch, dev, side, (ref_y, ref_s[0], *ref_s[1], ref_n), (y, ys, a, b, p, yn),
              "rwkv_wkv4_forward*")
        ws = rw.default_workspace("wkv4", dev, side)
        assert ws is not None
        assert rw.rwkv_wkv4_workspace_error(ws, stream=side) == 0


def test_wkv4_backward_and_training_pair_on_a_side_stream():
    torch, dev = torch_dev()
    t = _wkv4(torch)
    args = (t["w"], t["u"], t["k"], t["v"])
    ref = rw.rwkv_wkv4_backward(*args, t["gy"])
    B, T, C = t["k"].shape
    need = rw.rwkv_wkv4_backward_workspace(B, T, C)
    side = _side(torch, dev)
    for rep in range(2):
        log(f"wkv4 backward and training pair on a side stream, call {rep}")
        got = rw.rwkv_wkv4_backward(*args, t["gy"], stream=side)
        with torch.cuda.stream(side):
            ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        y = rw.rwkv_wkv4_forward_train(*args, ws, stream=side)
        pair = rw.rwkv_wkv4_backward_after_forward(*args, t["gy"], ws, stream=side)
        _same(torch, dev, side, (*ref, *ref), (*got, *pair), "rwkv_wkv4_backward*")
        assert torch.isfinite(y).all().item()


def test_wkv4_steps_on_a_side_stream():
    torch, dev = torch_dev()
    t = _wkv4(torch)
    B, T, C = t["k"].shape
    # per-token inputs made on the current stream before the side stream waits
    ks = [t["k"][:, s].contiguous() for s in range(20)]
    vs = [t["v"][:, s].contiguous() for s in range(20)]

    def run(stream):
        a, b, p = rw.rwkv_wkv4_state_init(B, C, device=dev, stream=stream)
        ys = [rw.rwkv_wkv4_step(a, b, p, t["w"], t["u"], ks[s], vs[s], stream=stream)
              for s in range(20)]
        return (*ys, a, b, p)

    ref = run(None)
    side = _side(torch, dev)
    log("wkv4 state init and 20 steps on a side stream")
    _same(torch, dev, side, ref, run(side), "rwkv_wkv4_step")


def test_matrix_state_entry_points_on_a_side_stream():
    torch, dev = torch_dev()
    e = synth.wkv6_inputs(2, 150, 3, 64, seed=32)
    bf = lambda n: to_dev(np.ascontiguousarray(e[n + "_bits"]), torch.bfloat16)  # noqa: E731
    r, k, v = bf("r"), bf("k"), bf("v")
    w, u, wt = to_dev(e["w"]), to_dev(e["u"]), to_dev(e["wt"])
    s0 = to_dev((np.random.default_rng(2).standard_normal((2, 3, 64, 64)) * 0.3)
                .astype(np.float32))
    # per-token inputs made on the current stream before the side stream waits
    tok = [tuple(x[:, t].contiguous() for x in (r, k, v, wt)) for t in range(5)]

    def run(stream):
        # the steps' states: written in full by a forward, then updated in place
        st5, st6 = (torch.empty((2, 3, 64, 64), dtype=torch.float32, device=dev)
                    for _ in range(2))
        o5 = rw.rwkv_wkv5_forward(r, k, v, w, u, stream=stream)
        o5s, s5 = rw.rwkv_wkv5_forward_state(r, k, v, w, u, s_in=s0, s_out=True, stream=stream)
        rw.rwkv_wkv5_forward_state(r, k, v, w, u, s_in=s0, s_out=st5, stream=stream)
        o6, s6 = rw.rwkv_wkv6_forward(r, k, v, wt, u, s_in=s0, s_out=True, stream=stream)
        rw.rwkv_wkv6_forward(r, k, v, wt, u, s_in=s0, s_out=st6, stream=stream)
        steps = []
        for rt, kt, vt, wtt in tok:
            steps.append(rw.rwkv_wkv5_step(st5, rt, kt, vt, w, u, stream=stream))
            steps.append(rw.rwkv_wkv6_step(st6, rt, kt, vt, wtt, u, stream=stream))
        return (o5, o5s, s5, o6, s6, *steps, st5, st6)

    ref = run(None)
    side = _side(torch, dev)
    for rep in range(2):
        log(f"Eagle and Finch forwards and steps on a side stream, call {rep}")
        _same(torch, dev, side, ref, run(side), "rwkv_wkv5/6")


def test_cached_workspace_is_zero_filled_again_when_its_count_comes_round(monkeypatch):
    """The binding zero-fills a cached RWKV-4 workspace again once it has
    served its period of calls (2^30; 3 here), before the call that finds the
    count come round: the workspace epoch (header word 1, one step per
    forward launch) then counts from that fill, and every call's y is the
    same."""
    torch, dev = torch_dev()
    monkeypatch.setattr(rw, "_WS_REZERO_EVERY", 3)
    t = _wkv4(torch)
    side = _side(torch, dev)
    ys = []
    for i in range(7):
        log(f"wkv4_forward call {i} on a fresh side stream (re-zero period 3)")
        ys.append(rw.rwkv_wkv4_forward(t["w"], t["u"], t["k"], t["v"], stream=side))
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    ws = rw.default_workspace("wkv4", dev, side)
    # fills before calls 0 (allocation), 3 and 6: one launch since the last
    assert ws.view(torch.int32)[1].item() == 1
    assert rw.rwkv_wkv4_workspace_error(ws, stream=side) == 0
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


@pytest.mark.parametrize("shape", [(8, 1024, 768), (1, 16384, 4096)])
def test_two_streams_run_forwards_at_once(shape):
    """Two streams, each with its own inputs and cached workspace, run RWKV-4
    forwards that overlap on the device (launch-order tiles at 8x1024x768,
    claimed tiles at 1x16384x4096): every output equals, bit for bit, the
    same call made alone on the current stream."""
    torch, dev = torch_dev()
    B, T, C = shape
    ins = []
    for seed in (61, 62):
        e = synth.wkv4_inputs(B, T, C, seed=seed)
        ins.append([to_dev(e[n]) for n in ("w", "u", "k", "v")])
    refs = [rw.rwkv_wkv4_forward(*a) for a in ins]
    torch.cuda.synchronize()
    streams = [_side(torch, dev), _side(torch, dev)]
    log(f"wkv4_forward {B}x{T}x{C} on two streams at once, 6 calls each")
    outs = [[], []]
    for _ in range(6):
        for j in (0, 1):
            outs[j].append(rw.rwkv_wkv4_forward(*ins[j], stream=streams[j]))
    for s in streams:
        torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    for j in (0, 1):
        ws = rw.default_workspace("wkv4", dev, streams[j])
        assert rw.rwkv_wkv4_workspace_error(ws, stream=streams[j]) == 0
        for y in outs[j]:
            assert torch.equal(y, refs[j])
