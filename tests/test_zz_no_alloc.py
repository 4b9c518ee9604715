"""The RWKV-4 forward that allocates nothing (rwkv_wkv4_forward_noalloc),
called through the C ABI, against rwkv_wkv4_forward on the same inputs:
the same kernels and plan, so the same bits, and both within the oracle's
bound.  Two calls in a row share the library's array, the second smaller
than the first (the array keeps the first call's words)."""
import ctypes

import numpy as np
import pytest

import linear_attention_sequence_rwkv_amd as rw
import oracle.wkv_oracle as O
import synth
from wkv_testutil import WKV4_TOL, log, torch_dev, wkv4_scaled_err

pytestmark = pytest.mark.gpu

WORKSPACE = -4


def _call_noalloc(lib, t, y, stream):
    B, T, C = t["k"].shape
    P = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731
    return lib.rwkv_wkv4_forward_noalloc(B, T, C, P(t["w"]), P(t["u"]), P(t["k"]), P(t["v"]),
                                         P(y), ctypes.c_void_p(stream.cuda_stream))


@pytest.mark.parametrize("order", ["big_then_small", "small_then_big_then_small"])
def test_noalloc_matches_the_workspace_forward(order):
    torch, dev = torch_dev()
    lib = rw.load_library()
    stream = torch.cuda.current_stream(dev)
    shapes = {"big_then_small": [(8, 1024, 768), (2, 300, 200)],
              "small_then_big_then_small": [(1, 70, 64), (4, 2048, 1024), (3, 1100, 200)]}[order]
    for i, (B, T, C) in enumerate(shapes):
        log(f"wkv4_forward_noalloc call {i}: B={B} T={T} C={C}")
        inp = synth.wkv4_inputs(B, T, C, seed=700 + i + T)
        t = {n: torch.from_numpy(inp[n]).to(dev) for n in ("w", "u", "k", "v")}
        y = torch.full((B, T, C), float("nan"), dtype=torch.float32, device=dev)
        assert _call_noalloc(lib, t, y, stream) == 0
        y_ws = rw.rwkv_wkv4_forward(t["w"], t["u"], t["k"], t["v"])
        torch.cuda.synchronize()
        assert torch.equal(y, y_ws)
        ch = np.arange(0, C, max(1, C // 24))
        y_ref, _ = O.wkv4_recurrent(inp["w"][ch], inp["u"][ch], inp["k"][..., ch],
                                    inp["v"][..., ch])
        S = O.wkv4_scale(inp["w"][ch], inp["u"][ch], inp["k"][..., ch], inp["v"][..., ch])
        err = wkv4_scaled_err(y.cpu().numpy()[..., ch], y_ref, S)
        log(f"  bitwise equal to rwkv_wkv4_forward; err vs oracle {err:.3e}")
        assert err <= WKV4_TOL


def test_noalloc_rejects_a_shape_beyond_its_array():
    """The long workload needs a 160 MB workspace: rejected, nothing launched
    (the pointers are real but far too small, and never touched)."""
    torch, dev = torch_dev()
    lib = rw.load_library()
    x = torch.zeros(64, dtype=torch.float32, device=dev)
    P = ctypes.c_void_p(x.data_ptr())
    st = lib.rwkv_wkv4_forward_noalloc(1, 65536, 5120, P, P, P, P, P,
                                       ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == WORKSPACE


def test_noalloc_replayed_from_a_captured_graph():
    """What the entry point is for: calls captured in a HIP graph (no
    allocation inside the capture) and replayed several times, with eager
    calls of other shapes on the same array in between.  Every replay equals
    the workspace forward on the replay's inputs, bit for bit."""
    torch, dev = torch_dev()
    lib = rw.load_library()
    shapes = [(2, 700, 128), (1, 1300, 192)]
    other = (3, 400, 320)
    bufs = [{n: torch.from_numpy(synth.wkv4_inputs(*shp, seed=800 + i)[n]).to(dev)
             for n in ("w", "u", "k", "v")} for i, shp in enumerate(shapes)]
    ys = [torch.empty_like(bf["k"]) for bf in bufs]
    o = {n: torch.from_numpy(x).to(dev)
         for n, x in synth.wkv4_inputs(*other, seed=810).items()}
    y_other = torch.empty_like(o["k"])
    cur = torch.cuda.current_stream(dev)
    assert _call_noalloc(lib, o, y_other, cur) == 0  # set-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(cur)
    with torch.cuda.graph(graph, stream=side):
        for bf, y in zip(bufs, ys):
            assert _call_noalloc(lib, bf, y, torch.cuda.current_stream(dev)) == 0
    torch.cuda.synchronize()
    for rnd in range(4):
        for i, (bf, shp) in enumerate(zip(bufs, shapes)):
            fresh = synth.wkv4_inputs(*shp, seed=820 + 10 * rnd + i)
            for n in ("w", "u", "k", "v"):
                bf[n].copy_(torch.from_numpy(fresh[n]))
        assert _call_noalloc(lib, o, y_other, cur) == 0  # eager, another shape, same array
        log(f"wkv4_forward_noalloc graph replay {rnd}")
        graph.replay()
        refs = [rw.rwkv_wkv4_forward(bf["w"], bf["u"], bf["k"], bf["v"]) for bf in bufs]
        torch.cuda.synchronize()
        for y, y_ref in zip(ys, refs):
            assert torch.equal(y, y_ref), rnd
