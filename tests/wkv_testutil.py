"""Shared helpers for the GPU parity tests (not collected by pytest)."""
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
