"""Shared helpers for the GPU parity tests (not collected by pytest)."""
import contextlib
import sys

import numpy as np


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def to_dev(x, dtype=None):
    torch, dev = torch_dev()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(dev)


def wkv4_scaled_err(y, y_ref, scale):
    """max |y - y_ref| / S, S the weighted mean of |v| (condition scale)."""
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(y - y_ref) / scale)) if y.size else 0.0


def wkv5_scaled_err(o, o_ref, o_abs):
    o = np.asarray(o, dtype=np.float64)
    return float(np.max(np.abs(o - o_ref) / np.maximum(o_abs, 1e-30))) if o.size else 0.0


WKV4_TOL = 1e-4
WKV5_TOL = 2e-2


def tile_code(tile):
    """RWKV_TUNE_WKV4_TILE value of a "cpl,L,NW" or "cpl,L,NW,CB" shape (CB:
    channel blocks per workgroup; None: the default plan)."""
    if tile is None:
        return 0
    parts = [int(x) for x in tile.split(",")]
    c, l, nw = parts[:3]
    cb = parts[3] if len(parts) > 3 else 1
    return (cb * 100000 if cb > 1 else 0) + c * 10000 + l * 100 + nw


@contextlib.contextmanager
def tuned(**settings):
    """Plan overrides for a block: wkv4_tile="cpl,L,NW", wkv4_claim=True,
    wkv5_dv=, wkv5_segs=, wkv6_dv=, wkv6_segs=, wkv4_spin= (None leaves a key alone)."""
    import linear_attention_sequence_rwkv_amd as rw
    keys = {"wkv4_tile": (rw.RWKV_TUNE_WKV4_TILE, tile_code),
            "wkv4_claim": (rw.RWKV_TUNE_WKV4_ORDER, lambda x: 1 if x else 0),
            "wkv5_dv": (rw.RWKV_TUNE_WKV5_DV, int),
            "wkv5_segs": (rw.RWKV_TUNE_WKV5_SEGS, int),
            "wkv6_dv": (rw.RWKV_TUNE_WKV6_DV, int),
            "wkv6_segs": (rw.RWKV_TUNE_WKV6_SEGS, int),
            "wkv4_spin": (rw.RWKV_TUNE_WKV4_SPIN, int)}
    with contextlib.ExitStack() as stack:
        for name, val in settings.items():
            if val is None:
                continue
            key, conv = keys[name]
            stack.enter_context(rw.tuning(key, conv(val)))
        yield
