#!/usr/bin/env python3
"""Benchmark of the RWKV WKV operators on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A "step" is one RWKV-4 WKV forward over the long-sequence workload
B=1 T=65536 C=5120 (the 14B-model width; float32 k, v, y; seeded synthetic
inputs already resident in HBM).  Its 4.03 GB working set is far larger than
the 256 MB Infinity Cache, so every step streams from HBM.  This is the
largest single-GPU workload of the forward, the one the time-parallel scan
exists for (few channels, a long sequence).

Printed: ONE JSON line.  `value` is achieved algorithmic HBM bandwidth
(12 bytes per element: read k, v; write y) over the K timed steps.
`roofline` relates the forward kernel's algorithmic bytes per launch to its
mean launch duration (two HIP events on the launch stream around K launches
back to back, one kernel per launch) and to the 8 TB/s HBM peak; `traffic`
is the HBM bytes per launch from the committed rocprofv3 counter summary
when that summary was taken on the current kernel source.  `cpu_baseline` is
the fp64 NumPy oracle on a channel sample of the same workload.  `secondary`
holds the other workloads and entry points, each timed as the median of five
repeats of at least 100 ms.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "WKV4 fwd achieved HBM GB/s (% of peak) + Gelem/s (B·T·C), fp32"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_attention_sequence_rwkv_amd", "csrc")
WKV4_SOURCES = ("wkv4.hip", "wkv4_scan.h", "wkv_device.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(files=WKV4_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_counter_summary(name: str, src_hash: str, key: str = "hbm_bytes_per_launch"):
    """A figure (HBM bytes per launch by default) from a committed rocprofv3
    counter summary, or None when the summary is missing or was taken on
    other kernel source.  The first line holding the key is used."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^\s*-?\s*`?(\w+)`?\s*[:=]\s*`?([0-9a-fA-F.eE+-]+)`?\s*$", line)
            if m and m.group(1) not in vals:
                vals[m.group(1)] = m.group(2)
    if vals.get("kernel_source_sha256") != src_hash:
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def measure(torch, stream, launch, calls_hint=1, min_ms=100.0, repeats=5):
    """Secondary-workload protocol: `launch(i)` enqueues call i on `stream`.
    The number of calls per repeat is raised until a repeat takes at least
    `min_ms`; returns (median ms per call, calls per repeat, all repeats)."""
    n = max(1, calls_hint)
    while True:
        s, e = _events(torch)
        s.record(stream)
        for i in range(n):
            launch(i)
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e)
        if ms >= min_ms or n >= 1 << 20:
            break
        n = max(n + 1, int(n * min_ms / max(ms, 1e-3) * 1.1))
    per = []
    for _ in range(repeats):
        s, e = _events(torch)
        s.record(stream)
        for i in range(n):
            launch(i)
        e.record(stream)
        torch.cuda.synchronize()
        per.append(s.elapsed_time(e) / n)
    return statistics.median(per), n, per


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------ RWKV-4 forward

def wkv4_device_copies(torch, inp, rotate):
    dev = torch.device("cuda:0")
    w = torch.from_numpy(inp["w"]).to(dev)
    u = torch.from_numpy(inp["u"]).to(dev)
    k0 = torch.from_numpy(inp["k"]).to(dev)
    v0 = torch.from_numpy(inp["v"]).to(dev)
    ks = [k0] + [k0.clone() for _ in range(rotate - 1)]
    vs = [v0] + [v0.clone() for _ in range(rotate - 1)]
    ys = [torch.empty_like(k0) for _ in range(rotate)]
    return w, u, ks, vs, ys


def wkv4_forward_calls(torch, rw, cfg, dev_inputs):
    """Pre-marshalled C-ABI argument tuples, one per rotated copy."""
    w, u, ks, vs, ys = dev_inputs
    B, T, C = cfg.B, cfg.T, cfg.C
    lib = rw.load_library()
    need = lib.rwkv_wkv4_forward_workspace(B, T, C)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=ks[0].device)
    stream = torch.cuda.current_stream(ks[0].device)
    sh = ctypes.c_void_p(stream.cuda_stream)
    calls = [(B, T, C, _ptr(w), _ptr(u), _ptr(ks[i]), _ptr(vs[i]), _ptr(ys[i]), _ptr(ws), need, sh)
             for i in range(len(ks))]
    return lib.rwkv_wkv4_forward, calls, stream, ws


def bench_wkv4_headline(torch, rw, cfg, dev_inputs, steps, warmup):
    """The driver's protocol: W untimed steps, then exactly K steps between
    two events (after a synchronisation on both sides)."""
    fn, calls, stream, ws = wkv4_forward_calls(torch, rw, cfg, dev_inputs)
    rot = len(calls)
    for i in range(warmup):
        assert fn(*calls[i % rot]) == 0
    torch.cuda.synchronize()
    s, e = _events(torch)
    s.record(stream)
    for i in range(steps):
        st = fn(*calls[i % rot])
        if st != 0:
            raise RuntimeError(f"rwkv_wkv4_forward status {st}")
    e.record(stream)
    torch.cuda.synchronize()
    total_ms = s.elapsed_time(e)
    _check_wkv4_output(torch, rw, dev_inputs, (steps - 1) % rot, ws)
    return total_ms / steps


def bench_wkv4_secondary(torch, rw, cfg, dev_inputs):
    fn, calls, stream, ws = wkv4_forward_calls(torch, rw, cfg, dev_inputs)
    rot = len(calls)
    for i in range(3):
        assert fn(*calls[i % rot]) == 0
    ms, n, per = measure(torch, stream, lambda i: fn(*calls[i % rot]), calls_hint=8)
    _check_wkv4_output(torch, rw, dev_inputs, (n - 1) % rot, ws)
    return ms, n, per


def _check_wkv4_output(torch, rw, dev_inputs, last, ws):
    """Sanity of the last launch: finite output, the first token is v, and
    the workspace's error word is clear."""
    _, _, ks, vs, ys = dev_inputs
    assert torch.isfinite(ys[last]).all().item()
    assert torch.equal(ys[last][:, 0], vs[last][:, 0])
    assert rw.rwkv_wkv4_workspace_error(ws) == 0


def copy_peak_gbps(torch, dev_inputs):
    """GB/s of the copy-peak kernel (y = a + b, 12 B per element, the RWKV-4
    forward's traffic with no dependencies; libwkv_copy_peak.so) over the
    same k, v, y buffers, rotated as the forward rotates them: >= 100 ms per
    repeat, median of 5.  None when that library has not been built."""
    path = os.path.join(ROOT, "linear_attention_sequence_rwkv_amd", "libwkv_copy_peak.so")
    if not os.path.exists(path):
        log("bench: libwkv_copy_peak.so missing (build() makes it); no copy peak")
        return None
    lib = ctypes.CDLL(path)
    lib.wkv_bench_add_copy.restype = ctypes.c_int
    lib.wkv_bench_add_copy.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]
    _, _, ks, vs, ys = dev_inputs
    rot = len(ks)
    n = ks[0].numel()
    stream = torch.cuda.current_stream(ks[0].device)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def launch(i):
        j = i % rot
        if lib.wkv_bench_add_copy(_ptr(ks[j]), _ptr(vs[j]), _ptr(ys[j]), n, sh) != 0:
            raise RuntimeError("wkv_bench_add_copy failed")

    for i in range(3):
        launch(i)
    ms, _, _ = measure(torch, stream, launch)
    return 12 * n / (ms * 1e-3) / 1e9


def wkv4_roofline(cfg, kern_ms, profile):
    nbytes = 12 * cfg.B * cfg.T * cfg.C
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    src = kernel_source_hash()
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": read_counter_summary(profile, src),
            "kernel": "wkv4_fwd_tiled", "kernel_us": round(kern_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": nbytes, "kernel_source": src}


def cpu_baseline_wkv4(cfg, inp, channels):
    """The fp64 oracle recurrence on the first `channels` channels of the
    same inputs over the full sequence (one host core: NumPy elementwise)."""
    import oracle.wkv_oracle as O
    sl = slice(0, channels)
    k, v = inp["k"][..., sl], inp["v"][..., sl]
    # whole passes until about 10 s of CPU work (at most 8)
    passes, el = 0, 0.0
    while passes < 8 and (passes == 0 or el < 10.0):
        t0 = time.perf_counter()
        O.wkv4_recurrent(inp["w"][sl], inp["u"][sl], k, v)
        el += time.perf_counter() - t0
        passes += 1
    el /= passes
    elems = cfg.B * cfg.T * channels
    return {"value": round(12 * elems / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"fp64 NumPy recurrence on channels 0..{channels - 1} of the "
                       f"{cfg.name} inputs (all {cfg.C}: the whole workload), full T={cfg.T}, "
                       f"{passes} pass(es) of {el:.1f} s each on one core of {_cpu_name()} "
                       f"({len(os.sched_getaffinity(0))} cores visible)"
                       if channels == cfg.C else
                       f"fp64 NumPy recurrence on channels 0..{channels - 1} of the "
                       f"{cfg.name} inputs, full T={cfg.T}, {passes} pass(es) of {el:.1f} s each "
                       f"on one core of {_cpu_name()} ({len(os.sched_getaffinity(0))} cores "
                       f"visible)"),
            "gelem_per_s": round(elems / el / 1e9, 6)}


# ------------------------------------------------------------------ others

def bench_wkv4_backward(torch, rw, cfg, rotate=1):
    """One backward call (prefix pass, reverse scan, reduction) per step,
    cycling over `rotate` copies of (k, v, gy) and of the gradients so that
    at 8x1024x768 the calls do not find their inputs in the 256 MB MALL."""
    import synth
    dev = torch.device("cuda:0")
    inp = synth.wkv4_backward_inputs(cfg.B, cfg.T, cfg.C, cfg.seed, omega_lo=cfg.omega_lo,
                                     omega_hi=cfg.omega_hi, u_std=cfg.u_std, k_std=cfg.k_std,
                                     v_std=cfg.v_std)
    B, T, C = cfg.B, cfg.T, cfg.C
    w, u = (torch.from_numpy(inp[n]).to(dev) for n in ("w", "u"))
    sets = []
    for _ in range(rotate):
        k, v, gy = (torch.from_numpy(inp[n]).to(dev) for n in ("k", "v", "gy"))
        sets.append((k, v, gy, torch.empty_like(k), torch.empty_like(k)))
    del inp
    gw, gu = torch.empty_like(w), torch.empty_like(u)
    lib = rw.load_library()
    need = lib.rwkv_wkv4_backward_workspace(B, T, C)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    args = [(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(gy), _ptr(gw), _ptr(gu), _ptr(gk),
             _ptr(gv), _ptr(ws), need, sh) for k, v, gy, gk, gv in sets]
    fn = lib.rwkv_wkv4_backward
    for i in range(2 * rotate):
        assert fn(*args[i % rotate]) == 0
    ms, n, _ = measure(torch, stream, lambda i: fn(*args[i % rotate]))
    for s in sets:
        assert torch.isfinite(s[3]).all().item() and torch.isfinite(s[4]).all().item()
    assert torch.isfinite(gw).all().item()
    assert rw.rwkv_wkv4_workspace_error(ws) == 0
    copy_gbps = None
    path = os.path.join(ROOT, "linear_attention_sequence_rwkv_amd", "libwkv_copy_peak.so")
    if os.path.exists(path):
        # the copy kernel with the backward's traffic, over the same buffers
        cl = ctypes.CDLL(path)
        cl.wkv_bench_three_two_copy.restype = ctypes.c_int
        cl.wkv_bench_three_two_copy.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_size_t,
                                                                        ctypes.c_void_p]

        def copy(i):
            k, v, gy, gk, gv = sets[i % rotate]
            if cl.wkv_bench_three_two_copy(_ptr(k), _ptr(v), _ptr(gy), _ptr(gk), _ptr(gv),
                                           B * T * C, sh) != 0:
                raise RuntimeError("wkv_bench_three_two_copy failed")

        for i in range(2 * rotate):
            copy(i)
        cms, _, _ = measure(torch, stream, copy)
        copy_gbps = 20 * B * T * C / (cms * 1e-3) / 1e9
    return {"ms": ms, "elems": B * T * C, "bytes": 20 * B * T * C, "calls_per_repeat": n,
            "copy_peak_GBps": copy_gbps, "rotated_copies": rotate}


def bench_wkv4_train(torch, rw, cfg, rotate=1):
    """A training step's WKV: forward then backward on the same inputs, timed
    as rwkv_wkv4_forward_train + rwkv_wkv4_backward_after_forward (one
    workspace, the backward reuses the forward's tile histories) and as
    rwkv_wkv4_forward + rwkv_wkv4_backward, cycling over `rotate` copies of
    the inputs and outputs as bench_wkv4_backward does."""
    import synth
    dev = torch.device("cuda:0")
    inp = synth.wkv4_backward_inputs(cfg.B, cfg.T, cfg.C, cfg.seed, omega_lo=cfg.omega_lo,
                                     omega_hi=cfg.omega_hi, u_std=cfg.u_std, k_std=cfg.k_std,
                                     v_std=cfg.v_std)
    B, T, C = cfg.B, cfg.T, cfg.C
    w, u = (torch.from_numpy(inp[n]).to(dev) for n in ("w", "u"))
    sets = []
    for _ in range(rotate):
        k, v, gy = (torch.from_numpy(inp[n]).to(dev) for n in ("k", "v", "gy"))
        sets.append((k, v, gy, torch.empty_like(k), torch.empty_like(k), torch.empty_like(k)))
    del inp
    gw, gu = torch.empty_like(w), torch.empty_like(u)
    lib = rw.load_library()
    need_b = lib.rwkv_wkv4_backward_workspace(B, T, C)
    need_f = lib.rwkv_wkv4_forward_workspace(B, T, C)
    ws_b = torch.zeros(max(need_b, 256), dtype=torch.uint8, device=dev)
    ws_f = torch.zeros(max(need_f, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    pair, separate = [], []
    for k, v, gy, y, gk, gv in sets:
        io = (_ptr(w), _ptr(u), _ptr(k), _ptr(v))
        grads = (_ptr(gy), _ptr(gw), _ptr(gu), _ptr(gk), _ptr(gv))
        pair.append(((lib.rwkv_wkv4_forward_train, (B, T, C, *io, _ptr(y), _ptr(ws_b), need_b, sh)),
                     (lib.rwkv_wkv4_backward_after_forward,
                      (B, T, C, *io, *grads, _ptr(ws_b), need_b, sh))))
        separate.append(((lib.rwkv_wkv4_forward, (B, T, C, *io, _ptr(y), _ptr(ws_f), need_f, sh)),
                         (lib.rwkv_wkv4_backward, (B, T, C, *io, *grads, _ptr(ws_b), need_b, sh))))
    out = {}
    for key, calls in (("pair", pair), ("separate", separate)):
        def launch(i, calls=calls):
            for fn, a in calls[i % rotate]:
                assert fn(*a) == 0
        for i in range(2 * rotate):
            launch(i)
        out[key], _, _ = measure(torch, stream, launch)
        for s in sets:
            assert torch.isfinite(s[3]).all().item() and torch.isfinite(s[4]).all().item()
    return {"ms": out["pair"], "ms_separate": out["separate"], "elems": B * T * C,
            "bytes": 32 * B * T * C, "rotated_copies": rotate}


def bench_decode(torch, rw, cfg, graph=True):
    """The 4096-step decode loop, eager and replayed from a HIP graph; one
    call of `launch` is one whole loop."""
    import synth
    dev = torch.device("cuda:0")
    inp = synth.wkv4_step_inputs(cfg.B, cfg.C, cfg.pool, cfg.seed)
    w = torch.from_numpy(inp["w"]).to(dev)
    u = torch.from_numpy(inp["u"]).to(dev)
    k_all = torch.from_numpy(inp["k"]).to(dev)
    v_all = torch.from_numpy(inp["v"]).to(dev)
    a, b, p = rw.rwkv_wkv4_state_init(cfg.B, cfg.C, device=dev)
    y = torch.empty((cfg.B, cfg.C), dtype=torch.float32, device=dev)
    lib = rw.load_library()

    def run(stream):
        sh = ctypes.c_void_p(stream.cuda_stream)
        for t in range(cfg.steps):
            i = t % cfg.pool
            st = lib.rwkv_wkv4_step(cfg.B, cfg.C, _ptr(a), _ptr(b), _ptr(p), _ptr(w), _ptr(u),
                                    _ptr(k_all[i]), _ptr(v_all[i]), _ptr(y), sh)
            if st != 0:
                raise RuntimeError(f"rwkv_wkv4_step status {st}")

    stream = torch.cuda.current_stream(dev)
    run(stream)  # warm-up
    torch.cuda.synchronize()
    eager_ms, _, _ = measure(torch, stream, lambda i: run(stream))
    elems = cfg.B * cfg.C * cfg.steps
    res = {"eager_ms": eager_ms, "graph_ms": None, "elems": elems, "bytes": 36 * elems}
    if graph:
        # The same 4096 launches captured once in a HIP graph and replayed.
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.graph(g, stream=cap):
            run(torch.cuda.current_stream(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        res["graph_ms"], _, _ = measure(torch, stream, lambda i: g.replay())
    assert torch.isfinite(y).all().item()
    return res


def bench_matrix_forward(torch, rw, cfg, finch, rotate=2):
    """Eagle (finch=False) or Finch forward; `rotate` copies of the inputs and
    output alternate so that consecutive calls do not find them in cache."""
    import synth
    dev = torch.device("cuda:0")
    e = (synth.wkv6_inputs(cfg.B, cfg.T, cfg.H, cfg.D, cfg.seed) if finch
         else synth.wkv5_inputs_for(cfg))
    to = lambda x: torch.from_numpy(x).to(dev)  # noqa: E731
    copies = []
    for _ in range(rotate):
        r, k, v = (to(e[n + "_bits"]).view(torch.bfloat16) for n in ("r", "k", "v"))
        wt = to(e["wt"]) if finch else None
        o = torch.empty((cfg.B, cfg.T, cfg.H, cfg.D), dtype=torch.float32, device=dev)
        copies.append((r, k, v, wt, o))
    w, u = to(e["w"]), to(e["u"])
    del e
    lib = rw.load_library()
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    query = lib.rwkv_wkv6_forward_workspace if finch else lib.rwkv_wkv5_forward_workspace
    need = query(cfg.B, cfg.T, cfg.H, cfg.D)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    shape = (cfg.B, cfg.T, cfg.H, cfg.D)
    if finch:
        calls = [(lib.rwkv_wkv6_forward, (*shape, _ptr(r), _ptr(k), _ptr(v), _ptr(wt), _ptr(u),
                                          _ptr(o), None, None, _ptr(ws), need, sh))
                 for r, k, v, wt, o in copies]
    else:
        calls = [(lib.rwkv_wkv5_forward, (*shape, _ptr(r), _ptr(k), _ptr(v), _ptr(w), _ptr(u),
                                          _ptr(o), _ptr(ws), need, sh))
                 for r, k, v, _, o in copies]

    def launch(i):
        fn, a = calls[i % rotate]
        assert fn(*a) == 0

    for i in range(2):
        launch(i)
    ms, n, _ = measure(torch, stream, launch, calls_hint=8)
    for c in copies:
        assert torch.isfinite(c[4]).all().item()
    elems = cfg.B * cfg.T * cfg.H * cfg.D
    nbytes = (14 if finch else 10) * elems
    copy_ms = mix_copy_ms(torch, copies, elems, stream)
    return {"ms": ms, "elems": elems, "bytes": nbytes,
            "flops": 4 * cfg.D * elems, "rotated_copies": rotate,
            "copy_peak_GBps": None if copy_ms is None else nbytes / (copy_ms * 1e-3) / 1e9}


def mix_copy_ms(torch, copies, elems, stream):
    """ms per call of the copy-peak kernel with the matrix-state forward's
    traffic (o = r + k + v [+ w_t], bf16 inputs, fp32 output: 10 or 14 B per
    element; libwkv_copy_peak.so) over the same rotated buffers: >= 100 ms
    per repeat, median of 5.  None when that library has not been built."""
    path = os.path.join(ROOT, "linear_attention_sequence_rwkv_amd", "libwkv_copy_peak.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.wkv_bench_mix_copy.restype = ctypes.c_int
    lib.wkv_bench_mix_copy.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p]
    sh = ctypes.c_void_p(stream.cuda_stream)

    def launch(i):
        r, k, v, wt, o = copies[i % len(copies)]
        wp = _ptr(wt) if wt is not None else None
        if lib.wkv_bench_mix_copy(_ptr(r), _ptr(k), _ptr(v), wp, _ptr(o), elems, sh) != 0:
            raise RuntimeError("wkv_bench_mix_copy failed")

    for i in range(3):
        launch(i)
    ms, _, _ = measure(torch, stream, launch)
    return ms


def wkv5_step_bytes(B, H, D):
    """Algorithmic bytes of one Eagle step: the fp32 state read and written,
    r, k, v in bf16, o in fp32."""
    return B * H * (2 * D * D * 4 + 3 * D * 2 + D * 4)


def bench_wkv5_decode(torch, rw, cfg):
    import synth
    dev = torch.device("cuda:0")
    inp = synth.wkv5_step_inputs(cfg)
    to = lambda x: torch.from_numpy(x).to(dev)  # noqa: E731
    # [B, pool, H, D] -> [pool, B, H, D]: one contiguous token per step
    r, k, v = (to(inp[n + "_bits"]).view(torch.bfloat16).transpose(0, 1).contiguous()
               for n in ("r", "k", "v"))
    w, u = to(inp["w"]), to(inp["u"])
    s = torch.zeros((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dev)
    o = torch.empty((cfg.B, cfg.H, cfg.D), dtype=torch.float32, device=dev)
    lib = rw.load_library()
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    calls = [(cfg.B, cfg.H, cfg.D, _ptr(s), _ptr(r[i]), _ptr(k[i]), _ptr(v[i]), _ptr(w), _ptr(u),
              _ptr(o), sh) for i in range(cfg.pool)]
    fn = lib.rwkv_wkv5_step

    def loop(_):
        for t in range(cfg.steps):
            assert fn(*calls[t % cfg.pool]) == 0

    loop(0)
    torch.cuda.synchronize()
    ms, _, _ = measure(torch, stream, loop)
    assert torch.isfinite(s).all().item()
    return {"ms": ms, "bytes": cfg.steps * wkv5_step_bytes(cfg.B, cfg.H, cfg.D)}


# ----------------------------------------------------- oracle samples (CPU)

def _cpu_name():
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return cpu


def cpu_sample_backward():
    """Oracle backward (reverse-time form) on 32 channels of the 8x1024x768
    workload, full T."""
    import oracle.wkv_oracle as O
    import synth
    cfg = synth.CFG_WKV4_169M
    inp = synth.wkv4_backward_inputs(cfg.B, cfg.T, 32, cfg.seed)
    t0 = time.perf_counter()
    O.wkv4_backward_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], inp["gy"])
    el = time.perf_counter() - t0
    elems = cfg.B * cfg.T * 32
    return {"value": round(20 * elems / el / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"B={cfg.B} T={cfg.T} x 32 channels, {el:.2f} s"}


def cpu_sample_decode():
    """Oracle steps for 16384 (stream, channel) lanes over 512 steps."""
    import numpy as np
    import oracle.wkv_oracle as O
    rng = np.random.default_rng(7)
    L, N = 16384, 512
    w = np.exp(rng.uniform(-3, 1, L)).astype(np.float32)
    u = (rng.standard_normal(L) * 0.5).astype(np.float32)
    k = rng.standard_normal((N, 1, L)).astype(np.float32)
    v = rng.standard_normal((N, 1, L)).astype(np.float32)
    st = O.wkv4_empty_state(1, L)
    t0 = time.perf_counter()
    for t in range(N):
        _, st = O.wkv4_step(st, w, u, k[t], v[t])
    el = time.perf_counter() - t0
    elems = L * N
    return {"value": round(36 * elems / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{L} lanes x {N} steps, {el:.1f} s"}


def cpu_sample_matrix(finch):
    """Oracle recurrence for 2 (batch, head) pairs over the full T."""
    import oracle.wkv_oracle as O
    import synth
    cfg = synth.CFG_WKV6_FINCH if finch else synth.CFG_WKV5_EAGLE
    t0 = time.perf_counter()
    if finch:
        e = synth.wkv6_inputs(1, cfg.T, 2, cfg.D, cfg.seed)
        t0 = time.perf_counter()
        O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"])
    else:
        e = synth.wkv5_inputs(1, cfg.T, 2, cfg.D, cfg.seed)
        t0 = time.perf_counter()
        O.wkv5_recurrent(e["r"], e["k"], e["v"], e["w"], e["u"])
    el = time.perf_counter() - t0
    elems = cfg.T * 2 * cfg.D
    return {"value": round((14 if finch else 10) * elems / el / 1e9, 5), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"2 heads x T={cfg.T} x D={cfg.D}, {el:.1f} s"}


def cpu_sample_eagle_decode():
    """Oracle steps for 4 (stream, head) pairs over all steps of the decode."""
    import numpy as np
    import oracle.wkv_oracle as O
    import synth
    cfg = synth.CFG_WKV5_DECODE
    inp = synth.wkv5_inputs(4, cfg.pool, 1, cfg.D, cfg.seed)
    S = np.zeros((4, 1, cfg.D, cfg.D))
    t0 = time.perf_counter()
    for t in range(cfg.steps):
        i = t % cfg.pool
        _, S = O.wkv5_step(S, inp["w"], inp["u"], inp["r"][:, i], inp["k"][:, i], inp["v"][:, i])
    el = time.perf_counter() - t0
    nbytes = cfg.steps * wkv5_step_bytes(4, 1, cfg.D)
    return {"value": round(nbytes / el / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"4 (stream, head) pairs x {cfg.steps} steps, {el:.2f} s"}


def cpu_sample_169m():
    """The fp64 oracle recurrence over the full 8x1024x768 workload, once."""
    import oracle.wkv_oracle as O
    import synth
    cfg = synth.CFG_WKV4_169M
    inp = synth.wkv4_inputs_for(cfg)
    t0 = time.perf_counter()
    O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
    el = time.perf_counter() - t0
    elems = cfg.B * cfg.T * cfg.C
    return {"value": round(12 * elems / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": f"the full workload, {el:.1f} s"}


# --------------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB three times with torch (a plain copy of known "
                         "size, for scaling the HBM byte counters of a rocprofv3 run)")
    ap.add_argument("--cpu-channels", type=int, default=5120,
                    help="channels of the headline workload the oracle sample covers")
    ap.add_argument("--secondary",
                    default="169m,169m-hot,decode,decode-graph,eagle,eagle-wide,eagle-decode,"
                            "finch,backward,backward-long,train,long-steady",
                    help="comma list of secondary workloads: 169m, 169m-hot, decode, "
                         "decode-graph, eagle, eagle-wide, eagle-decode, finch, backward, "
                         "backward-long, train, long-steady (the headline workload "
                         "itself, run last)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the operator shards over batch/channels with no communication); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import linear_attention_sequence_rwkv_amd as rw
    import synth
    rw.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.copy_calibration:
        a = torch.ones((1 << 28,), dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()

    # The headline's inputs are made (host work of several seconds) and put
    # in device memory first; the secondary workloads run next and the
    # headline last, so that its W warmup and K timed steps follow busy
    # seconds of GPU work: after an idle spell the device's clocks take about
    # 15 ms of load to settle, over which the first launches run up to 5%
    # slower.
    cfg = synth.CFG_WKV4_LONG
    inp = synth.wkv4_inputs_for(cfg)
    dev_inputs = wkv4_device_copies(torch, inp, rotate=1)

    want = set() if args.no_secondary else {x for x in args.secondary.split(",") if x}
    sec = {}
    if "169m" in want or "169m-hot" in want:
        c2 = synth.CFG_WKV4_169M
        i2 = synth.wkv4_inputs_for(c2)
        for key, rot in (("169m", 5), ("169m-hot", 1)):
            if key not in want:
                continue
            log(f"bench: {c2.name} rotating {rot} cop{'ies' if rot > 1 else 'y'}")
            d2 = wkv4_device_copies(torch, i2, rot)
            ms2, n2, per2 = bench_wkv4_secondary(torch, rw, c2, d2)
            cp2 = copy_peak_gbps(torch, d2) if rot > 1 else None
            del d2
            name = c2.name if rot > 1 else c2.name + "_hot"
            g = 12 * c2.B * c2.T * c2.C / (ms2 * 1e-3) / 1e9
            sec[name] = {"ms": round(ms2, 5), "GBps": round(g, 1),
                         "gelem_per_s": round(c2.B * c2.T * c2.C / (ms2 * 1e-3) / 1e9, 1),
                         "rotated_copies": rot, "calls_per_repeat": n2,
                         "repeats_ms": [round(x, 5) for x in per2]}
            if rot > 1:
                sec[name]["roofline"] = wkv4_roofline(c2, ms2, "wkv4_fwd_tiled_B8_T1024_C768.md")
                if cp2 is not None:
                    sec[name]["copy_peak_GBps"] = round(cp2, 1)
                    sec[name]["pct_of_copy_peak"] = round(100 * g / cp2, 2)
    if "decode" in want or "decode-graph" in want:
        dc = synth.CFG_WKV4_DECODE
        log(f"bench: {dc.name}")
        r = bench_decode(torch, rw, dc, graph="decode-graph" in want)
        d = {"eager_ms": round(r["eager_ms"], 3),
             "eager_GBps": round(r["bytes"] / (r["eager_ms"] * 1e-3) / 1e9, 1),
             "us_per_step_eager": round(1e3 * r["eager_ms"] / dc.steps, 3),
             "bytes_per_elem_step": 36,
             "note": "effective bandwidth: the 12.6 MB state can stay in the 256 MB MALL"}
        if r["graph_ms"] is not None:
            d.update({"graph_ms": round(r["graph_ms"], 3),
                      "graph_GBps": round(r["bytes"] / (r["graph_ms"] * 1e-3) / 1e9, 1),
                      "us_per_step_graph": round(1e3 * r["graph_ms"] / dc.steps, 3)})
        sec[dc.name] = d
    if "eagle-decode" in want:
        ed = synth.CFG_WKV5_DECODE
        log(f"bench: {ed.name}")
        r = bench_wkv5_decode(torch, rw, ed)
        sec[ed.name] = {"ms": round(r["ms"], 4),
                        "us_per_step": round(1e3 * r["ms"] / ed.steps, 3),
                        "GBps": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 1),
                        "note": "effective bandwidth: the 32 MB state can stay in the MALL"}
    for key, mc, finch in (("eagle", synth.CFG_WKV5_EAGLE, False),
                           ("eagle-wide", synth.CFG_WKV5_EAGLE_WIDE, False),
                           ("finch", synth.CFG_WKV6_FINCH, True)):
        if key not in want:
            continue
        log(f"bench: {mc.name}")
        r = bench_matrix_forward(torch, rw, mc, finch)
        hsrc = kernel_source_hash(("wkv6.hip" if finch else "wkv5.hip", "eagle_common.h",
                                   "wkv_device.h"))
        prof = (("wkv6" if finch else "wkv5") + "_fwd_chunked_mfma_B4_T4096_H32_D64.md")
        g = r["bytes"] / (r["ms"] * 1e-3) / 1e9
        cp = r["copy_peak_GBps"]
        sec[mc.name] = {"ms": round(r["ms"], 4),
                        "GBps": round(g, 1),
                        "bytes_per_elem": 14 if finch else 10,
                        "copy_peak_GBps": None if cp is None else round(cp, 1),
                        "pct_of_copy_peak": None if cp is None else round(100 * g / cp, 2),
                        "algorithmic_TFLOPs": round(r["flops"] / (r["ms"] * 1e-3) / 1e12, 2),
                        "mfma_busy_pct": read_counter_summary(
                            prof, hsrc, "mfma_busy_pct_wide" if key == "eagle-wide"
                            else "mfma_busy_pct"),
                        "rotated_copies": r["rotated_copies"]}
    def backward(key, bc, rotate):
        if key in want:
            name = bc.name.replace("wkv4_fwd", "wkv4_bwd")
            log(f"bench: {name}")
            r = bench_wkv4_backward(torch, rw, bc, rotate)
            g = r["bytes"] / (r["ms"] * 1e-3) / 1e9
            cp = r["copy_peak_GBps"]
            sec[name] = {"ms": round(r["ms"], 5),
                         "GBps": round(g, 1),
                         "bytes_per_elem": 20,
                         "copy_peak_GBps": None if cp is None else round(cp, 1),
                         "pct_of_copy_peak": None if cp is None else round(100 * g / cp, 2),
                         "gelem_per_s": round(r["elems"] / (r["ms"] * 1e-3) / 1e9, 1),
                         "rotated_copies": r["rotated_copies"]}

    backward("backward", synth.CFG_WKV4_169M, 6)
    if "train" in want:
        tc = synth.CFG_WKV4_169M
        name = tc.name.replace("wkv4_fwd", "wkv4_train_step")
        log(f"bench: {name}")
        r = bench_wkv4_train(torch, rw, tc, 6)
        sec[name] = {"ms": round(r["ms"], 5),
                     "ms_forward_plus_backward": round(r["ms_separate"], 5),
                     "GBps": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 1),
                     "bytes_per_elem": 32, "rotated_copies": r["rotated_copies"]}
    backward("backward-long", synth.CFG_WKV4_LONG, 1)
    if "long-steady" in want:
        # The headline workload under the secondary protocol, last before the
        # headline: its steady-state rate, and K timed steps that start on a
        # device already running this kernel.
        name = cfg.name + "_steady"
        log(f"bench: {name}")
        ms3, n3, per3 = bench_wkv4_secondary(torch, rw, cfg, dev_inputs)
        sec[name] = {"ms": round(ms3, 5),
                     "GBps": round(12 * cfg.B * cfg.T * cfg.C / (ms3 * 1e-3) / 1e9, 1),
                     "rotated_copies": 1, "calls_per_repeat": n3,
                     "repeats_ms": [round(x, 5) for x in per3]}

    log(f"bench: {cfg.name} steps={args.steps} warmup={args.warmup}")
    ms = bench_wkv4_headline(torch, rw, cfg, dev_inputs, args.steps, args.warmup)
    log("bench: copy peak on the same buffers")
    copy_peak = copy_peak_gbps(torch, dev_inputs)
    del dev_inputs
    torch.cuda.empty_cache()
    nbytes = 12 * cfg.B * cfg.T * cfg.C
    value = nbytes / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "C": cfg.C,
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
                   "gelem_per_s": round(cfg.B * cfg.T * cfg.C / (ms * 1e-3) / 1e9, 2),
                   "bytes_per_elem": 12, "rotated_copies": 1,
                   "after_secondary_workloads": bool(sec),
                   "copy_peak_GBps": None if copy_peak is None else round(copy_peak, 1),
                   "pct_of_copy_peak": (None if copy_peak is None
                                        else round(100 * value / copy_peak, 2))},
        # one kernel per step, launched back to back: the step time is the
        # kernel's mean duration plus the sub-microsecond launch gap
        "roofline": wkv4_roofline(cfg, ms, "wkv4_fwd_tiled_B1_T65536_C5120.md"),
    }
    if sec:
        line["secondary"] = sec

    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline_wkv4(cfg, inp, min(args.cpu_channels, cfg.C))
        samplers = {synth.CFG_WKV4_169M.name: cpu_sample_169m,
                    synth.CFG_WKV4_DECODE.name: cpu_sample_decode,
                    synth.CFG_WKV5_EAGLE.name: lambda: cpu_sample_matrix(False),
                    synth.CFG_WKV5_DECODE.name: cpu_sample_eagle_decode,
                    synth.CFG_WKV6_FINCH.name: lambda: cpu_sample_matrix(True),
                    synth.CFG_WKV4_169M.name.replace("wkv4_fwd", "wkv4_bwd"):
                        cpu_sample_backward}
        for name, fn in samplers.items():
            if name in sec:
                sec[name]["cpu_baseline"] = fn()

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
