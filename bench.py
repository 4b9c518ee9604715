#!/usr/bin/env python3
"""Benchmark of the RWKV WKV operators on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A "step" is one RWKV-4 WKV forward over the workload B=8 T=1024 C=768
(float32 k, v, y; seeded synthetic inputs already resident in HBM).  Five
copies of (k, v, y) rotate so that the 377 MB working set exceeds
the 256 MB Infinity Cache and every step reads from HBM.

Printed: ONE JSON line.  `value` is achieved algorithmic HBM bandwidth
(12 bytes per element: read k, v; write y) over the timed steps.
`roofline` relates the forward kernel's algorithmic bytes per launch to its
mean launch duration (HIP events around every launch, on the launch stream)
and to the 8 TB/s HBM peak.  `cpu_baseline` is the fp64 NumPy oracle timed
on this host on the same workload.  `secondary` holds the other entry points
(long-sequence forward, the 4096-step decode loop, the Eagle forward).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import re
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(files=("wkv4.hip", "wkv4_scan.h", "wkv_device.h")) -> str:
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


class Timer:
    """A pair of HIP events bracketing the timed region on one stream."""

    def __init__(self, torch):
        E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        self.start, self.end = E(), E()


def bench_wkv4_forward(torch, rw, cfg, steps, warmup, rotate):
    import synth
    dev = torch.device("cuda:0")
    inp = synth.wkv4_inputs_for(cfg)
    B, T, C = cfg.B, cfg.T, cfg.C
    w = torch.from_numpy(inp["w"]).to(dev)
    u = torch.from_numpy(inp["u"]).to(dev)
    k0 = torch.from_numpy(inp["k"]).to(dev)
    v0 = torch.from_numpy(inp["v"]).to(dev)
    ks = [k0] + [k0.clone() for _ in range(rotate - 1)]
    vs = [v0] + [v0.clone() for _ in range(rotate - 1)]
    ys = [torch.empty_like(k0) for _ in range(rotate)]
    lib = rw.load_library()
    need = lib.rwkv_wkv4_forward_workspace(B, T, C)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    # Marshalled once; the timed loop is nothing but C-ABI calls.
    calls = [(B, T, C, P(w), P(u), P(ks[i]), P(vs[i]), P(ys[i]), P(ws), need, sh)
             for i in range(rotate)]
    fn = lib.rwkv_wkv4_forward
    for i in range(warmup):
        assert fn(*calls[i % rotate]) == 0
    torch.cuda.synchronize()
    # Timed region: K launches back to back, bracketed by two events.
    tm = Timer(torch)
    tm.start.record(stream)
    for i in range(steps):
        st = fn(*calls[i % rotate])
        if st != 0:
            raise RuntimeError(f"rwkv_wkv4_forward status {st}")
    tm.end.record(stream)
    torch.cuda.synchronize()
    total_ms = tm.start.elapsed_time(tm.end)
    # One kernel per call, launched back to back on this stream: its average
    # duration is the timed region over K.  (An event pair around each launch
    # would add the event packets' own dispatch gaps to every launch.)
    kern_ms = total_ms / steps
    # sanity: the output of the last launch is finite and the first token is v
    y_last = ys[(steps - 1) % rotate]
    assert torch.isfinite(y_last).all().item()
    assert torch.equal(y_last[:, 0], vs[(steps - 1) % rotate][:, 0])
    return {"ms_per_step": total_ms / steps, "kernel_ms": kern_ms,
            "elems": B * T * C, "bytes": 12 * B * T * C}


def bench_wkv4_backward(torch, rw, cfg, steps, warmup):
    """One backward call (prefix pass, reverse scan, reduction) per step."""
    import synth
    dev = torch.device("cuda:0")
    inp = synth.wkv4_backward_inputs(cfg.B, cfg.T, cfg.C, cfg.seed, omega_lo=cfg.omega_lo,
                                     omega_hi=cfg.omega_hi, u_std=cfg.u_std, k_std=cfg.k_std,
                                     v_std=cfg.v_std)
    B, T, C = cfg.B, cfg.T, cfg.C
    w, u, k, v, gy = (torch.from_numpy(inp[n]).to(dev) for n in ("w", "u", "k", "v", "gy"))
    gw, gu = torch.empty_like(w), torch.empty_like(u)
    gk, gv = torch.empty_like(k), torch.empty_like(k)
    lib = rw.load_library()
    need = lib.rwkv_wkv4_backward_workspace(B, T, C)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    args = (B, T, C, P(w), P(u), P(k), P(v), P(gy), P(gw), P(gu), P(gk), P(gv), P(ws), need,
            ctypes.c_void_p(stream.cuda_stream))
    fn = lib.rwkv_wkv4_backward
    for _ in range(warmup):
        assert fn(*args) == 0
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record(stream)
    for _ in range(steps):
        assert fn(*args) == 0
    en.record(stream)
    torch.cuda.synchronize()
    assert torch.isfinite(gk).all().item() and torch.isfinite(gw).all().item()
    ms = st.elapsed_time(en) / steps
    return {"ms": ms, "elems": B * T * C, "bytes": 20 * B * T * C}


def bench_wkv4_train(torch, rw, cfg, steps, warmup):
    """A training step's WKV: forward then backward on the same inputs, timed
    as rwkv_wkv4_forward_train + rwkv_wkv4_backward_after_forward (one
    workspace, the backward reuses the forward's tile histories) and as
    rwkv_wkv4_forward + rwkv_wkv4_backward."""
    import synth
    dev = torch.device("cuda:0")
    inp = synth.wkv4_backward_inputs(cfg.B, cfg.T, cfg.C, cfg.seed, omega_lo=cfg.omega_lo,
                                     omega_hi=cfg.omega_hi, u_std=cfg.u_std, k_std=cfg.k_std,
                                     v_std=cfg.v_std)
    B, T, C = cfg.B, cfg.T, cfg.C
    w, u, k, v, gy = (torch.from_numpy(inp[n]).to(dev) for n in ("w", "u", "k", "v", "gy"))
    y = torch.empty_like(k)
    gw, gu = torch.empty_like(w), torch.empty_like(u)
    gk, gv = torch.empty_like(k), torch.empty_like(k)
    lib = rw.load_library()
    need_b = lib.rwkv_wkv4_backward_workspace(B, T, C)
    need_f = lib.rwkv_wkv4_forward_workspace(B, T, C)
    ws_b = torch.zeros(max(need_b, 256), dtype=torch.uint8, device=dev)
    ws_f = torch.zeros(max(need_f, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    io = (P(w), P(u), P(k), P(v))
    grads = (P(gy), P(gw), P(gu), P(gk), P(gv))
    pair = ((lib.rwkv_wkv4_forward_train, (B, T, C, *io, P(y), P(ws_b), need_b, sh)),
            (lib.rwkv_wkv4_backward_after_forward, (B, T, C, *io, *grads, P(ws_b), need_b, sh)))
    separate = ((lib.rwkv_wkv4_forward, (B, T, C, *io, P(y), P(ws_f), need_f, sh)),
                (lib.rwkv_wkv4_backward, (B, T, C, *io, *grads, P(ws_b), need_b, sh)))
    out = {}
    for key, calls in (("pair", pair), ("separate", separate)):
        for _ in range(warmup):
            for fn, a in calls:
                assert fn(*a) == 0
        torch.cuda.synchronize()
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record(stream)
        for _ in range(steps):
            for fn, a in calls:
                assert fn(*a) == 0
        en.record(stream)
        torch.cuda.synchronize()
        assert torch.isfinite(gk).all().item() and torch.isfinite(y).all().item()
        out[key] = st.elapsed_time(en) / steps
    return {"ms": out["pair"], "ms_separate": out["separate"], "elems": B * T * C,
            "bytes": 32 * B * T * C}


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


def bench_copy_peak(torch, nbytes=1 << 30, reps=20):
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    return 2 * nbytes / (ms * 1e-3) / 1e9


def bench_decode(torch, rw, cfg, reps, graph=True):
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
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def run(stream):
        sh = ctypes.c_void_p(stream.cuda_stream)
        for t in range(cfg.steps):
            i = t % cfg.pool
            st = lib.rwkv_wkv4_step(cfg.B, cfg.C, P(a), P(b), P(p), P(w), P(u), P(k_all[i]),
                                    P(v_all[i]), P(y), sh)
            if st != 0:
                raise RuntimeError(f"rwkv_wkv4_step status {st}")

    stream = torch.cuda.current_stream(dev)
    run(stream)  # warm-up
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        run(stream)
    e.record(stream)
    torch.cuda.synchronize()
    eager_ms = s.elapsed_time(e) / reps
    elems = cfg.B * cfg.C * cfg.steps
    if not graph:
        assert torch.isfinite(y).all().item()
        return {"eager_ms": eager_ms, "graph_ms": None, "elems": elems, "bytes": 36 * elems}
    # The same 4096 launches captured once in a HIP graph and replayed.
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    with torch.cuda.graph(g, stream=cap):
        run(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    s.record(stream)
    for _ in range(reps):
        g.replay()
    e.record(stream)
    torch.cuda.synchronize()
    graph_ms = s.elapsed_time(e) / reps
    assert torch.isfinite(y).all().item()
    return {"eager_ms": eager_ms, "graph_ms": graph_ms, "elems": elems, "bytes": 36 * elems}


def bench_wkv5(torch, rw, cfg, reps):
    import synth
    dev = torch.device("cuda:0")
    inp = synth.wkv5_inputs_for(cfg)
    to = lambda x: torch.from_numpy(x).to(dev)  # noqa: E731
    r, k, v = (to(inp[n + "_bits"]).view(torch.bfloat16) for n in ("r", "k", "v"))
    w, u = to(inp["w"]), to(inp["u"])
    o = torch.empty((cfg.B, cfg.T, cfg.H, cfg.D), dtype=torch.float32, device=dev)
    lib = rw.load_library()
    need = lib.rwkv_wkv5_forward_workspace(cfg.B, cfg.T, cfg.H, cfg.D)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    args = (cfg.B, cfg.T, cfg.H, cfg.D, P(r), P(k), P(v), P(w), P(u), P(o), P(ws), need,
            ctypes.c_void_p(stream.cuda_stream))
    assert lib.rwkv_wkv5_forward(*args) == 0
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        assert lib.rwkv_wkv5_forward(*args) == 0
    e.record(stream)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item()
    ms = s.elapsed_time(e) / reps
    elems = cfg.B * cfg.T * cfg.H * cfg.D
    return {"ms": ms, "elems": elems, "bytes": 10 * elems, "flops": 4 * cfg.D * elems}


def bench_wkv6(torch, rw, cfg, reps):
    import synth
    dev = torch.device("cuda:0")
    e = synth.wkv6_inputs(cfg.B, cfg.T, cfg.H, cfg.D, cfg.seed)
    to = lambda x: torch.from_numpy(x).to(dev)  # noqa: E731
    r, k, v = (to(e[n + "_bits"]).view(torch.bfloat16) for n in ("r", "k", "v"))
    wt, u = to(e["wt"]), to(e["u"])
    o = torch.empty((cfg.B, cfg.T, cfg.H, cfg.D), dtype=torch.float32, device=dev)
    lib = rw.load_library()
    stream = torch.cuda.current_stream(dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    need = lib.rwkv_wkv6_forward_workspace(cfg.B, cfg.T, cfg.H, cfg.D)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    args = (cfg.B, cfg.T, cfg.H, cfg.D, P(r), P(k), P(v), P(wt), P(u), P(o), None, None, P(ws),
            need, ctypes.c_void_p(stream.cuda_stream))
    assert lib.rwkv_wkv6_forward(*args) == 0
    torch.cuda.synchronize()
    s, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        assert lib.rwkv_wkv6_forward(*args) == 0
    en.record(stream)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item()
    ms = s.elapsed_time(en) / reps
    elems = cfg.B * cfg.T * cfg.H * cfg.D
    return {"ms": ms, "elems": elems, "bytes": 14 * elems, "flops": 4 * cfg.D * elems}


def cpu_sample_finch():
    """Oracle recurrence for 2 (batch, head) pairs over the full T."""
    import oracle.wkv_oracle as O
    import synth
    cfg = synth.CFG_WKV6_FINCH
    e = synth.wkv6_inputs(1, cfg.T, 2, cfg.D, cfg.seed)
    t0 = time.perf_counter()
    O.wkv6_recurrent(e["r"], e["k"], e["v"], e["wt"], e["u"])
    el = time.perf_counter() - t0
    elems = cfg.T * 2 * cfg.D
    return {"value": round(14 * elems / el / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"2 heads x T={cfg.T} x D={cfg.D}, {el:.1f} s"}


def wkv5_step_bytes(B, H, D):
    """Algorithmic bytes of one Eagle step: the fp32 state read and written,
    r, k, v in bf16, o in fp32."""
    return B * H * (2 * D * D * 4 + 3 * D * 2 + D * 4)


def bench_wkv5_decode(torch, rw, cfg, reps):
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
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    calls = [(cfg.B, cfg.H, cfg.D, P(s), P(r[i]), P(k[i]), P(v[i]), P(w), P(u), P(o), sh)
             for i in range(cfg.pool)]
    fn = lib.rwkv_wkv5_step
    for i in range(8):
        assert fn(*calls[i % cfg.pool]) == 0
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record(stream)
        for t in range(cfg.steps):
            assert fn(*calls[t % cfg.pool]) == 0
        en.record(stream)
        torch.cuda.synchronize()
        ms = st.elapsed_time(en)
        best = ms if best is None else min(best, ms)
    assert torch.isfinite(s).all().item()
    return {"ms": best, "bytes": cfg.steps * wkv5_step_bytes(cfg.B, cfg.H, cfg.D)}


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


def cpu_sample_long(budget_s=4.0):
    """Oracle on channels of the long-sequence workload, over the full T."""
    import numpy as np
    import oracle.wkv_oracle as O
    import synth
    cfg = synth.CFG_WKV4_LONG
    inp = synth.wkv4_inputs(1, cfg.T, 64, cfg.seed, omega_lo=cfg.omega_lo, omega_hi=cfg.omega_hi,
                            u_std=cfg.u_std, k_std=cfg.k_std)
    t0 = time.perf_counter()
    O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
    el = time.perf_counter() - t0
    elems = cfg.T * 64
    del np
    return {"value": round(12 * elems / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"64 channels x T={cfg.T} of the same distributions, {el:.1f} s"}


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


def cpu_sample_eagle():
    """Oracle recurrence for 2 (batch, head) pairs over the full T."""
    import oracle.wkv_oracle as O
    import synth
    cfg = synth.CFG_WKV5_EAGLE
    inp = synth.wkv5_inputs(1, cfg.T, 2, cfg.D, cfg.seed)
    t0 = time.perf_counter()
    O.wkv5_recurrent(inp["r"], inp["k"], inp["v"], inp["w"], inp["u"])
    el = time.perf_counter() - t0
    elems = cfg.T * 2 * cfg.D
    return {"value": round(10 * elems / el / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
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


def cpu_baseline(cfg, budget_s):
    """The fp64 oracle's recurrence on the full workload, repeated for about
    `budget_s` seconds of host time."""
    import numpy as np
    import oracle.wkv_oracle as O
    import synth
    inp = synth.wkv4_inputs_for(cfg)
    reps, t0 = 0, time.perf_counter()
    while True:
        O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    elems = cfg.B * cfg.T * cfg.C * reps
    cpu = _cpu_name()
    del np
    return {"value": round(12 * elems / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"fp64 NumPy recurrence over the full B={cfg.B} T={cfg.T} C={cfg.C} "
                       f"workload, {reps} run(s) in {el:.1f} s on one core of {cpu} "
                       f"({len(os.sched_getaffinity(0))} cores visible)"),
            "gelem_per_s": round(elems / el / 1e9, 6)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=5)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="accepted for older command lines; the 1 GiB copy always runs")
    ap.add_argument("--secondary",
                    default="hot,long,decode,decode-graph,eagle,eagle-decode,finch,backward,"
                            "backward-long,train",
                    help="comma list of secondary workloads: hot, long, decode, decode-graph, "
                         "eagle, eagle-decode, finch, backward, backward-long, train")
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

    cfg = synth.CFG_WKV4_169M
    copy_gbps = bench_copy_peak(torch)
    log(f"bench: {cfg.name} steps={args.steps} warmup={args.warmup} rotate={args.rotate}")
    prim = bench_wkv4_forward(torch, rw, cfg, args.steps, args.warmup, args.rotate)
    value = prim["bytes"] / (prim["ms_per_step"] * 1e-3) / 1e9
    achieved = prim["bytes"] / (prim["kernel_ms"] * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = read_counter_summary("wkv4_fwd_tiled_B8_T1024_C768.md", src_hash)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "C": cfg.C,
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
                   "pct_of_copy_peak": round(100 * value / copy_gbps, 2),
                   "gelem_per_s": round(prim["elems"] / (prim["ms_per_step"] * 1e-3) / 1e9, 2),
                   "bytes_per_elem": 12, "rotated_copies": args.rotate},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "wkv4_fwd_tiled",
                     "kernel_us": round(prim["kernel_ms"] * 1e3, 3),
                     "kernel_source": src_hash},
    }
    line["copy_peak_GBps"] = round(copy_gbps, 1)

    want = set() if args.no_secondary else {x for x in args.secondary.split(",") if x}
    if want:
        sec = {}
        if "hot" in want:
            log(f"bench: {cfg.name} hot (one copy of k, v, y)")
            r = bench_wkv4_forward(torch, rw, cfg, steps=args.steps, warmup=args.warmup, rotate=1)
            sec[cfg.name + "_hot"] = {
                "ms": round(r["ms_per_step"], 5), "kernel_ms": round(r["kernel_ms"], 5),
                "GBps": round(r["bytes"] / (r["ms_per_step"] * 1e-3) / 1e9, 1)}
        if "long" in want:
            lc = synth.CFG_WKV4_LONG
            log(f"bench: {lc.name}")
            r = bench_wkv4_forward(torch, rw, lc, steps=10, warmup=2, rotate=1)
            sec[lc.name] = {"ms": round(r["ms_per_step"], 4),
                            "kernel_ms": round(r["kernel_ms"], 4),
                            "GBps": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 1),
                            "gelem_per_s": round(r["elems"] / (r["kernel_ms"] * 1e-3) / 1e9, 1)}
        if "decode" in want or "decode-graph" in want:
            dc = synth.CFG_WKV4_DECODE
            log(f"bench: {dc.name}")
            r = bench_decode(torch, rw, dc, reps=3, graph="decode-graph" in want)
            d = {"eager_ms": round(r["eager_ms"], 3),
                 "eager_GBps": round(r["bytes"] / (r["eager_ms"] * 1e-3) / 1e9, 1)}
            if r["graph_ms"] is not None:
                d.update({"graph_ms": round(r["graph_ms"], 3),
                          "graph_GBps": round(r["bytes"] / (r["graph_ms"] * 1e-3) / 1e9, 1),
                          "us_per_step_graph": round(1e3 * r["graph_ms"] / dc.steps, 3)})
            sec[dc.name] = d
        if "eagle" in want:
            ec = synth.CFG_WKV5_EAGLE
            log(f"bench: {ec.name}")
            r = bench_wkv5(torch, rw, ec, reps=5)
            sec[ec.name] = {"ms": round(r["ms"], 4),
                            "GBps": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 1),
                            "algorithmic_TFLOPs": round(r["flops"] / (r["ms"] * 1e-3) / 1e12, 2),
                            "mfma_busy_pct": read_counter_summary(
                                "wkv5_fwd_chunked_mfma_B4_T4096_H32_D64.md",
                                kernel_source_hash(("wkv5.hip", "eagle_common.h", "wkv_device.h")),
                                "mfma_busy_pct")}
        for key, bc, n_steps in (("backward", cfg, 100), ("backward-long", synth.CFG_WKV4_LONG, 3)):
            if key in want:
                name = bc.name.replace("wkv4_fwd", "wkv4_bwd")
                log(f"bench: {name}")
                r = bench_wkv4_backward(torch, rw, bc, steps=n_steps, warmup=2)
                sec[name] = {"ms": round(r["ms"], 5),
                             "GBps": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 1),
                             "bytes_per_elem": 20,
                             "gelem_per_s": round(r["elems"] / (r["ms"] * 1e-3) / 1e9, 1)}
        if "train" in want:
            name = cfg.name.replace("wkv4_fwd", "wkv4_train_step")
            log(f"bench: {name}")
            r = bench_wkv4_train(torch, rw, cfg, steps=100, warmup=2)
            sec[name] = {"ms": round(r["ms"], 5),
                         "ms_forward_plus_backward": round(r["ms_separate"], 5),
                         "GBps": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 1),
                         "bytes_per_elem": 32}
        if "finch" in want:
            fc = synth.CFG_WKV6_FINCH
            log(f"bench: {fc.name}")
            r = bench_wkv6(torch, rw, fc, reps=5)
            sec[fc.name] = {"ms": round(r["ms"], 4),
                            "GBps": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 1),
                            "bytes_per_elem": 14,
                            "algorithmic_TFLOPs": round(r["flops"] / (r["ms"] * 1e-3) / 1e12, 2),
                            "mfma_busy_pct": read_counter_summary(
                                "wkv6_fwd_chunked_mfma_B4_T4096_H32_D64.md",
                                kernel_source_hash(("wkv6.hip", "eagle_common.h", "wkv_device.h")),
                                "mfma_busy_pct")}
        if "eagle-decode" in want:
            ed = synth.CFG_WKV5_DECODE
            log(f"bench: {ed.name}")
            r = bench_wkv5_decode(torch, rw, ed, reps=3)
            sec[ed.name] = {"ms": round(r["ms"], 4),
                            "us_per_step": round(1e3 * r["ms"] / ed.steps, 3),
                            "GBps": round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 1)}
        line["secondary"] = sec

    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
        sec = line.get("secondary", {})
        samplers = {synth.CFG_WKV4_LONG.name: cpu_sample_long,
                    synth.CFG_WKV4_DECODE.name: cpu_sample_decode,
                    synth.CFG_WKV5_EAGLE.name: cpu_sample_eagle,
                    synth.CFG_WKV5_DECODE.name: cpu_sample_eagle_decode,
                    synth.CFG_WKV6_FINCH.name: cpu_sample_finch,
                    synth.CFG_WKV4_169M.name.replace("wkv4_fwd", "wkv4_bwd"): cpu_sample_backward}
        for name, fn in samplers.items():
            if name in sec:
                sec[name]["cpu_baseline"] = fn()

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
