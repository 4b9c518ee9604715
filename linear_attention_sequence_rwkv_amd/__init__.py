"""Python binding of librwkv_wkv.so: the RWKV WKV operators on MI355X.

Argument marshalling only.  Each function has the name of the C entry point
it calls (declared in include/rwkv_wkv.h), takes torch tensors that already
live on the GPU, passes their device pointers and torch's current HIP stream,
and turns a negative status into an exception.  Every step of the
computation runs in the library's HIP kernels; there is no fallback: if the
library is missing, every call raises.

torch is used only to allocate outputs/workspaces and to name the stream.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "LIB_PATH", "load_library", "RwkvError",
    "rwkv_abi_version", "rwkv_status_str", "rwkv_last_hip_error",
    "RWKV_TUNE_WKV4_TILE", "RWKV_TUNE_WKV4_ORDER", "RWKV_TUNE_WKV5_DV",
    "RWKV_TUNE_WKV5_SEGS", "RWKV_TUNE_WKV6_DV", "RWKV_TUNE_WKV6_SEGS", "RWKV_TUNE_WKV4_SPIN",
    "rwkv_set_tuning", "rwkv_get_tuning", "tuning",
    "rwkv_wkv4_workspace_error",
    "rwkv_wkv4_forward_workspace", "rwkv_wkv4_forward", "rwkv_wkv4_forward_state",
    "rwkv_wkv4_forward_noalloc",
    "rwkv_wkv4_backward_workspace", "rwkv_wkv4_backward",
    "rwkv_wkv4_forward_train", "rwkv_wkv4_backward_after_forward",
    "rwkv_wkv4_state_init", "rwkv_wkv4_step",
    "rwkv_wkv5_forward_workspace", "rwkv_wkv5_forward", "rwkv_wkv5_forward_state",
    "rwkv_wkv5_step",
    "rwkv_wkv6_forward_workspace", "rwkv_wkv6_forward", "rwkv_wkv6_step",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librwkv_wkv.so")

_lib = None
_lib_lock = threading.Lock()

_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_p = ctypes.c_void_p

# name -> (restype, argtypes), mirroring include/rwkv_wkv.h
_SIGNATURES = {
    "rwkv_abi_version": (ctypes.c_int, []),
    "rwkv_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "rwkv_last_hip_error": (ctypes.c_int, []),
    "rwkv_set_tuning": (ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
    "rwkv_get_tuning": (ctypes.c_int, [ctypes.c_int]),
    "rwkv_wkv4_workspace_error": (ctypes.c_int, [_p, _sz, _p, _p]),
    "rwkv_wkv4_forward_workspace": (_sz, [_i64, _i64, _i64]),
    "rwkv_wkv4_forward_noalloc": (ctypes.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p]),
    "rwkv_wkv4_forward": (ctypes.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "rwkv_wkv4_forward_state": (ctypes.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _p,
                                               _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "rwkv_wkv4_backward_workspace": (_sz, [_i64, _i64, _i64]),
    "rwkv_wkv4_backward": (ctypes.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                          _p, _sz, _p]),
    "rwkv_wkv4_forward_train": (ctypes.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _sz,
                                               _p]),
    "rwkv_wkv4_backward_after_forward": (ctypes.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p,
                                                        _p, _p, _p, _p, _sz, _p]),
    "rwkv_wkv4_state_init": (ctypes.c_int, [_i64, _i64, _p, _p, _p, _p]),
    "rwkv_wkv4_step": (ctypes.c_int, [_i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "rwkv_wkv5_forward_workspace": (_sz, [_i64, _i64, _i64, _i64]),
    "rwkv_wkv5_forward": (ctypes.c_int,
                          [_i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "rwkv_wkv5_forward_state": (ctypes.c_int, [_i64, _i64, _i64, _i64, _p, _p, _p, _p, _p,
                                               _p, _p, _p, _p, _sz, _p]),
    "rwkv_wkv5_step": (ctypes.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p]),
    "rwkv_wkv6_forward_workspace": (_sz, [_i64, _i64, _i64, _i64]),
    "rwkv_wkv6_forward": (ctypes.c_int, [_i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p,
                                         _p, _sz, _p]),
    "rwkv_wkv6_step": (ctypes.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p]),
}


class RwkvError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str, hip_error: int = 0):
        super().__init__(f"{fn}: status {status} ({msg})"
                         + (f", hipError {hip_error}" if hip_error else ""))
        self.status = status
        self.hip_error = hip_error


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise ImportError(
                f"{p} not found: build it with "
                "`python -m linear_attention_sequence_rwkv_amd.build`")
        lib = ctypes.CDLL(p)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _check(fn: str, status: int) -> None:
    if status == 0:
        return
    lib = load_library()
    msg = lib.rwkv_status_str(status).decode()
    if status == -6:
        raise RwkvError(fn, status, msg, lib.rwkv_last_hip_error())
    raise ValueError(f"{fn}: status {status} ({msg})")


def rwkv_abi_version() -> int:
    return load_library().rwkv_abi_version()


def rwkv_status_str(status: int) -> str:
    return load_library().rwkv_status_str(status).decode()


def rwkv_last_hip_error() -> int:
    return load_library().rwkv_last_hip_error()


# Plan override keys (include/rwkv_wkv.h).
RWKV_TUNE_WKV4_TILE = 1
RWKV_TUNE_WKV4_ORDER = 2
RWKV_TUNE_WKV5_DV = 3
RWKV_TUNE_WKV5_SEGS = 4
RWKV_TUNE_WKV6_DV = 5
RWKV_TUNE_WKV6_SEGS = 6
RWKV_TUNE_WKV4_SPIN = 7


def rwkv_set_tuning(key: int, value: int) -> None:
    _check("rwkv_set_tuning", load_library().rwkv_set_tuning(key, value))


def rwkv_get_tuning(key: int) -> int:
    return int(load_library().rwkv_get_tuning(key))


class tuning:
    """Context manager: a plan override for the duration of a block, e.g.
    ``with tuning(RWKV_TUNE_WKV5_DV, 32): ...`` (the previous value returns
    afterwards)."""

    def __init__(self, key: int, value: int):
        self.key, self.value, self.old = key, value, None

    def __enter__(self):
        self.old = rwkv_get_tuning(self.key)
        rwkv_set_tuning(self.key, self.value)
        return self

    def __exit__(self, *exc):
        rwkv_set_tuning(self.key, self.old)
        return False


# ---------------------------------------------------------------- helpers ---

def _torch():
    import torch
    return torch


def _dev_tensor(name, t, dtypes, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _launch_stream(device, stream=None):
    """(torch stream, handle) of the stream the library call is enqueued on."""
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s, ctypes.c_void_p(s.cuda_stream)


def _use_on(stream, *tensors):
    """A call on a stream other than torch's current one: tell torch's
    allocator that these tensors are in use there until that stream's work
    is done (outputs the binding allocates are allocated on `stream` itself,
    see _alloc)."""
    torch = _torch()
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _alloc(stream, fn, *args, **kw):
    """Allocate (and fill) a tensor with torch on `stream`, so that its
    memory is ordered with the library call enqueued there."""
    torch = _torch()
    with torch.cuda.stream(stream):
        return fn(*args, **kw)


# Workspaces are zero-filled once and reused per (device, stream): the
# library leaves them ready for the next call on the same stream.  The fill
# and the allocation happen on that stream, ahead of the call.  The RWKV-4
# workspaces tag their words with a 32-bit count of launches (a call makes at
# most two), so a cached one is zero-filled again every 2^30 calls, at the
# first call made outside graph capture once the count has come round.
_ws_cache: dict = {}
_ws_calls: dict = {}
_ws_lock = threading.Lock()
_WS_REZERO_EVERY = 1 << 30


def _workspace(kind: str, device, stream, nbytes: int):
    if nbytes == 0:
        return None
    torch = _torch()
    key = (kind, device.index, stream.cuda_stream)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = _alloc(stream, torch.zeros, max(nbytes, 1 << 16), dtype=torch.uint8,
                         device=device)
            _ws_cache[key] = buf
            _ws_calls[key] = 0
        elif _ws_calls[key] >= _WS_REZERO_EVERY and not _alloc(
                stream, torch.cuda.is_current_stream_capturing):
            _alloc(stream, buf.zero_)
            _ws_calls[key] = 0
        _ws_calls[key] += 1
        return buf


def rwkv_wkv4_workspace_error(ws, stream=None) -> int:
    """The error word of an RWKV-4 workspace (0: no device-side error since
    it was zero-filled).  Synchronises ``stream`` (default: the current one)."""
    torch = _torch()
    lib = load_library()
    ws = _dev_tensor("ws", ws, (torch.uint8,))
    s, sh = _launch_stream(ws.device, stream)
    out = _alloc(s, torch.zeros, 1, dtype=torch.int32, device=ws.device)
    _check("rwkv_wkv4_workspace_error",
           lib.rwkv_wkv4_workspace_error(_ptr(ws), ws.numel(), _ptr(out), sh))
    s.synchronize()
    return int(out.item()) & 0xFFFFFFFF


def default_workspace(kind: str, device, stream=None):
    """The workspace the binding keeps for (kind, device, stream), or None;
    kind is one of "wkv4", "wkv4_bwd", "wkv5", "wkv6"."""
    torch = _torch()
    dev = torch.device(device)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with _ws_lock:
        return _ws_cache.get((kind, dev.index, s.cuda_stream))


# ----------------------------------------------------------------- RWKV-4 ---
#
# Every entry point enqueues on ``stream`` (default: torch's current stream).
# Outputs the binding allocates, and its cached workspaces, are allocated (and
# zero-filled) on that stream, so they are ordered with the call; with an
# explicit stream that is not the current one, every tensor argument is
# recorded on it for torch's allocator.  Inputs written on another stream must
# be made visible to ``stream`` by the caller, as for any torch work on a side
# stream.

def rwkv_wkv4_forward_workspace(B: int, T: int, C: int) -> int:
    return int(load_library().rwkv_wkv4_forward_workspace(B, T, C))


def _wkv4_inputs(w, u, k, v):
    torch = _torch()
    f32 = (torch.float32,)
    k = _dev_tensor("k", k, f32, 3)
    v = _dev_tensor("v", v, f32, 3)
    w = _dev_tensor("w", w, f32, 1)
    u = _dev_tensor("u", u, f32, 1)
    B, T, C = k.shape
    if tuple(v.shape) != (B, T, C) or w.shape[0] != C or u.shape[0] != C:
        raise ValueError("shape mismatch among w, u, k, v")
    return w, u, k, v


def _out(name, t, shape, device, s):
    """A float32 output: allocated on the launch stream, or the caller's
    tensor checked for shape."""
    torch = _torch()
    if t is None:
        return _alloc(s, torch.empty, shape, dtype=torch.float32, device=device)
    t = _dev_tensor(name, t, (torch.float32,), len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has the wrong shape")
    return t


def _wkv4_ws(lib, k, ws, s):
    B, T, C = k.shape
    need = lib.rwkv_wkv4_forward_workspace(B, T, C)
    if ws is None:
        ws = _workspace("wkv4", k.device, s, need)
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def rwkv_wkv4_forward(w, u, k, v, y=None, ws=None, stream=None):
    """y[B,T,C] = WKV(w, u, k, v); see rwkv_wkv4_forward in rwkv_wkv.h.

    ``ws`` (optional) is a caller-owned zero-initialised uint8 GPU tensor of at
    least rwkv_wkv4_forward_workspace(B, T, C) bytes; by default a cached one
    per (device, stream) is used.
    """
    lib = load_library()
    w, u, k, v = _wkv4_inputs(w, u, k, v)
    B, T, C = k.shape
    s, sh = _launch_stream(k.device, stream)
    y = _out("y", y, (B, T, C), k.device, s)
    ws, nbytes = _wkv4_ws(lib, k, ws, s)
    _use_on(stream, w, u, k, v, y, ws)
    status = lib.rwkv_wkv4_forward(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                   _ptr(ws), nbytes, sh)
    _check("rwkv_wkv4_forward", status)
    return y


def rwkv_wkv4_forward_noalloc(w, u, k, v, y=None, stream=None):
    """rwkv_wkv4_forward with the library's own workspace (nothing allocated
    by the library; ``y`` is allocated here if not given)."""
    lib = load_library()
    w, u, k, v = _wkv4_inputs(w, u, k, v)
    B, T, C = k.shape
    s, sh = _launch_stream(k.device, stream)
    y = _out("y", y, (B, T, C), k.device, s)
    _use_on(stream, w, u, k, v, y)
    status = lib.rwkv_wkv4_forward_noalloc(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                           sh)
    _check("rwkv_wkv4_forward_noalloc", status)
    return y


def _wkv4_state_args(name, state, B, C):
    torch = _torch()
    if len(state) != 3:
        raise ValueError(f"{name} must be a triple (a, b, p)")
    out = tuple(_dev_tensor(f"{name}[{i}]", t, (torch.float32,), 2) for i, t in enumerate(state))
    for t in out:
        if tuple(t.shape) != (B, C):
            raise ValueError(f"{name} arrays must be [B, C] = [{B}, {C}]")
    return out


def rwkv_wkv4_forward_state(w, u, k, v, state_in=None, state_out=None, y=None, ws=None,
                            stream=None):
    """Forward from the history ``state_in`` (a, b, p) or empty if None.

    ``state_out``: None (final state not wanted), True (allocate), or a triple
    of float32 [B, C] tensors to write (may be ``state_in`` itself).  Returns
    (y, state_out).
    """
    torch = _torch()
    lib = load_library()
    w, u, k, v = _wkv4_inputs(w, u, k, v)
    B, T, C = k.shape
    s, sh = _launch_stream(k.device, stream)
    y = _out("y", y, (B, T, C), k.device, s)
    sin = (None, None, None) if state_in is None else _wkv4_state_args("state_in", state_in, B, C)
    if state_out is True:
        state_out = tuple(_alloc(s, torch.empty, (B, C), dtype=torch.float32, device=k.device)
                          for _ in range(3))
    sout = (None, None, None) if state_out is None else _wkv4_state_args("state_out", state_out,
                                                                        B, C)
    ws, nbytes = _wkv4_ws(lib, k, ws, s)
    _use_on(stream, w, u, k, v, y, ws, *sin, *sout)
    status = lib.rwkv_wkv4_forward_state(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                         *(_ptr(t) for t in sin), *(_ptr(t) for t in sout),
                                         _ptr(ws), nbytes, sh)
    _check("rwkv_wkv4_forward_state", status)
    return y, (None if state_out is None else sout)


def rwkv_wkv4_backward_workspace(B: int, T: int, C: int) -> int:
    return int(load_library().rwkv_wkv4_backward_workspace(B, T, C))


def rwkv_wkv4_backward(w, u, k, v, gy, gw=None, gu=None, gk=None, gv=None, ws=None,
                       stream=None, _entry="rwkv_wkv4_backward"):
    """Gradients of sum(gy * WKV(w, u, k, v)).  Returns (gw, gu, gk, gv).

    ``ws`` (optional) is a caller-owned zero-initialised uint8 GPU tensor of at
    least rwkv_wkv4_backward_workspace(B, T, C) bytes; by default a cached one
    per (device, stream) is used.
    """
    torch = _torch()
    lib = load_library()
    w, u, k, v = _wkv4_inputs(w, u, k, v)
    B, T, C = k.shape
    gy = _dev_tensor("gy", gy, (torch.float32,), 3)
    if tuple(gy.shape) != (B, T, C):
        raise ValueError("gy has the wrong shape")
    s, sh = _launch_stream(k.device, stream)
    gw, gu = _out("gw", gw, (C,), k.device, s), _out("gu", gu, (C,), k.device, s)
    gk, gv = _out("gk", gk, (B, T, C), k.device, s), _out("gv", gv, (B, T, C), k.device, s)
    need = lib.rwkv_wkv4_backward_workspace(B, T, C)
    if ws is None:
        if _entry != "rwkv_wkv4_backward":
            raise ValueError("rwkv_wkv4_backward_after_forward needs the workspace that "
                             "rwkv_wkv4_forward_train used")
        ws = _workspace("wkv4_bwd", k.device, s, need)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _use_on(stream, w, u, k, v, gy, gw, gu, gk, gv, ws)
    status = getattr(lib, _entry)(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(gy),
                                  _ptr(gw), _ptr(gu), _ptr(gk), _ptr(gv), _ptr(ws), nbytes, sh)
    _check(_entry, status)
    return gw, gu, gk, gv


def rwkv_wkv4_forward_train(w, u, k, v, ws, y=None, stream=None):
    """The forward for training: returns y as rwkv_wkv4_forward does and leaves
    in ``ws`` (a zero-initialised uint8 GPU tensor of at least
    rwkv_wkv4_backward_workspace(B, T, C) bytes) the tile histories that
    rwkv_wkv4_backward_after_forward reads instead of recomputing."""
    lib = load_library()
    w, u, k, v = _wkv4_inputs(w, u, k, v)
    B, T, C = k.shape
    if ws is None:
        raise ValueError("rwkv_wkv4_forward_train needs a backward workspace")
    s, sh = _launch_stream(k.device, stream)
    y = _out("y", y, (B, T, C), k.device, s)
    nbytes = ws.numel() * ws.element_size()
    _use_on(stream, w, u, k, v, y, ws)
    status = lib.rwkv_wkv4_forward_train(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                         _ptr(ws), nbytes, sh)
    _check("rwkv_wkv4_forward_train", status)
    return y


def rwkv_wkv4_backward_after_forward(w, u, k, v, gy, ws, gw=None, gu=None, gk=None, gv=None,
                                     stream=None):
    """rwkv_wkv4_backward's gradients, reusing the histories that the last
    rwkv_wkv4_forward_train over the same inputs left in ``ws``."""
    return rwkv_wkv4_backward(w, u, k, v, gy, gw, gu, gk, gv, ws, stream,
                              _entry="rwkv_wkv4_backward_after_forward")


def rwkv_wkv4_state_init(B: int, C: int, device="cuda", stream=None):
    """Return an empty recurrent state (a, b, p), three float32 [B, C] tensors."""
    torch = _torch()
    lib = load_library()
    dev = torch.device(device)
    s, sh = _launch_stream(dev, stream)
    a, b, p = (_alloc(s, torch.empty, (B, C), dtype=torch.float32, device=dev)
               for _ in range(3))
    status = lib.rwkv_wkv4_state_init(B, C, _ptr(a), _ptr(b), _ptr(p), sh)
    _check("rwkv_wkv4_state_init", status)
    return a, b, p


def rwkv_wkv4_step(a, b, p, w, u, k, v, y=None, stream=None):
    """One token: returns y[B,C] and updates the state (a, b, p) in place."""
    torch = _torch()
    lib = load_library()
    f32 = (torch.float32,)
    a, b, p = (_dev_tensor(n, t, f32, 2) for n, t in (("a", a), ("b", b), ("p", p)))
    k = _dev_tensor("k", k, f32, 2)
    v = _dev_tensor("v", v, f32, 2)
    w = _dev_tensor("w", w, f32, 1)
    u = _dev_tensor("u", u, f32, 1)
    B, C = a.shape
    for n, t in (("b", b), ("p", p), ("k", k), ("v", v)):
        if tuple(t.shape) != (B, C):
            raise ValueError(f"{n} has the wrong shape")
    if w.shape[0] != C or u.shape[0] != C:
        raise ValueError("w, u must have C entries")
    s, sh = _launch_stream(a.device, stream)
    y = _out("y", y, (B, C), a.device, s)
    _use_on(stream, a, b, p, w, u, k, v, y)
    status = lib.rwkv_wkv4_step(B, C, _ptr(a), _ptr(b), _ptr(p), _ptr(w), _ptr(u), _ptr(k),
                                _ptr(v), _ptr(y), sh)
    _check("rwkv_wkv4_step", status)
    return y


# ------------------------------------------------------------------ Eagle ---

def rwkv_wkv5_forward_workspace(B: int, T: int, H: int, D: int) -> int:
    return int(load_library().rwkv_wkv5_forward_workspace(B, T, H, D))


def _wkv5_args(r, k, v, w, u, ndim):
    torch = _torch()
    half = (torch.bfloat16, torch.int16, torch.uint16)
    r = _dev_tensor("r", r, half, ndim)
    k = _dev_tensor("k", k, half, ndim)
    v = _dev_tensor("v", v, half, ndim)
    if w is not None:  # None: the caller checks a per-token decay itself
        w = _dev_tensor("w", w, (torch.float32,), 2)
    u = _dev_tensor("u", u, (torch.float32,), 2)
    shape = tuple(r.shape)
    H, D = shape[-2], shape[-1]
    if tuple(k.shape) != shape or tuple(v.shape) != shape:
        raise ValueError("r, k, v shapes differ")
    if (w is not None and tuple(w.shape) != (H, D)) or tuple(u.shape) != (H, D):
        raise ValueError("w, u must be [H, D]")
    return r, k, v, w, u


def _ws(kind, query, shape, device, ws, s):
    need = query(*shape)
    if ws is None:
        ws = _workspace(kind, device, s, need)
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def rwkv_wkv5_forward(r, k, v, w, u, o=None, ws=None, stream=None):
    """o[B,T,H,D] float32 from bf16 r, k, v [B,T,H,D] and float32 w, u [H,D]."""
    lib = load_library()
    r, k, v, w, u = _wkv5_args(r, k, v, w, u, 4)
    B, T, H, D = r.shape
    s, sh = _launch_stream(r.device, stream)
    o = _out("o", o, (B, T, H, D), r.device, s)
    ws, nbytes = _ws("wkv5", lib.rwkv_wkv5_forward_workspace, (B, T, H, D), r.device, ws, s)
    _use_on(stream, r, k, v, w, u, o, ws)
    status = lib.rwkv_wkv5_forward(B, T, H, D, _ptr(r), _ptr(k), _ptr(v), _ptr(w), _ptr(u),
                                   _ptr(o), _ptr(ws), nbytes, sh)
    _check("rwkv_wkv5_forward", status)
    return o


def _wkv5_state_arg(name, st, B, H, D):
    torch = _torch()
    st = _dev_tensor(name, st, (torch.float32,), 4)
    if tuple(st.shape) != (B, H, D, D):
        raise ValueError(f"{name} must be [B, H, D, D] = [{B}, {H}, {D}, {D}]")
    return st


def _state_out(s_out, B, H, D, device, s):
    torch = _torch()
    if s_out is True:
        return _alloc(s, torch.empty, (B, H, D, D), dtype=torch.float32, device=device)
    if s_out is not None:
        return _wkv5_state_arg("s_out", s_out, B, H, D)
    return None


def rwkv_wkv5_forward_state(r, k, v, w, u, s_in=None, s_out=None, o=None, ws=None,
                            stream=None):
    """Eagle forward from the state ``s_in`` [B,H,D,D] (zero if None).

    ``s_out``: None (not wanted), True (allocate) or a float32 [B,H,D,D]
    tensor (may be ``s_in``).  Returns (o, s_out).
    """
    lib = load_library()
    r, k, v, w, u = _wkv5_args(r, k, v, w, u, 4)
    B, T, H, D = r.shape
    s, sh = _launch_stream(r.device, stream)
    o = _out("o", o, (B, T, H, D), r.device, s)
    if s_in is not None:
        s_in = _wkv5_state_arg("s_in", s_in, B, H, D)
    s_out = _state_out(s_out, B, H, D, r.device, s)
    ws, nbytes = _ws("wkv5", lib.rwkv_wkv5_forward_workspace, (B, T, H, D), r.device, ws, s)
    _use_on(stream, r, k, v, w, u, o, ws, s_in, s_out)
    status = lib.rwkv_wkv5_forward_state(B, T, H, D, _ptr(r), _ptr(k), _ptr(v), _ptr(w),
                                         _ptr(u), _ptr(o), _ptr(s_in), _ptr(s_out), _ptr(ws),
                                         nbytes, sh)
    _check("rwkv_wkv5_forward_state", status)
    return o, s_out


def rwkv_wkv5_step(s, r, k, v, w, u, o=None, stream=None):
    """One Eagle token: r, k, v [B,H,D] bf16; s [B,H,D,D] updated in place.

    Returns o [B,H,D] float32.
    """
    lib = load_library()
    r, k, v, w, u = _wkv5_args(r, k, v, w, u, 3)
    B, H, D = r.shape
    st = _wkv5_state_arg("s", s, B, H, D)
    ls, sh = _launch_stream(r.device, stream)
    o = _out("o", o, (B, H, D), r.device, ls)
    _use_on(stream, st, r, k, v, w, u, o)
    status = lib.rwkv_wkv5_step(B, H, D, _ptr(st), _ptr(r), _ptr(k), _ptr(v), _ptr(w), _ptr(u),
                                _ptr(o), sh)
    _check("rwkv_wkv5_step", status)
    return o


# ------------------------------------------------------------------ Finch ---

def _finch_w(w, shape):
    torch = _torch()
    w = _dev_tensor("w", w, (torch.float32,), len(shape))
    if tuple(w.shape) != shape:
        raise ValueError(f"w must have the shape of r, {shape}")
    return w


def rwkv_wkv6_forward_workspace(B: int, T: int, H: int, D: int) -> int:
    return int(load_library().rwkv_wkv6_forward_workspace(B, T, H, D))


def rwkv_wkv6_forward(r, k, v, w, u, s_in=None, s_out=None, o=None, ws=None, stream=None):
    """Finch forward: r, k, v [B,T,H,D] bf16, w [B,T,H,D] float32 per-token
    decays, u [H,D].  ``s_in``/``s_out`` as for rwkv_wkv5_forward_state.
    Returns (o, s_out)."""
    lib = load_library()
    r, k, v, _, u = _wkv5_args(r, k, v, None, u, 4)
    B, T, H, D = r.shape
    w = _finch_w(w, (B, T, H, D))
    s, sh = _launch_stream(r.device, stream)
    o = _out("o", o, (B, T, H, D), r.device, s)
    if s_in is not None:
        s_in = _wkv5_state_arg("s_in", s_in, B, H, D)
    s_out = _state_out(s_out, B, H, D, r.device, s)
    ws, nbytes = _ws("wkv6", lib.rwkv_wkv6_forward_workspace, (B, T, H, D), r.device, ws, s)
    _use_on(stream, r, k, v, w, u, o, ws, s_in, s_out)
    status = lib.rwkv_wkv6_forward(B, T, H, D, _ptr(r), _ptr(k), _ptr(v), _ptr(w), _ptr(u),
                                   _ptr(o), _ptr(s_in), _ptr(s_out), _ptr(ws), nbytes, sh)
    _check("rwkv_wkv6_forward", status)
    return o, s_out


def rwkv_wkv6_step(s, r, k, v, w, u, o=None, stream=None):
    """One Finch token: r, k, v [B,H,D] bf16, w [B,H,D] float32; s updated in
    place.  Returns o [B,H,D] float32."""
    lib = load_library()
    r, k, v, _, u = _wkv5_args(r, k, v, None, u, 3)
    B, H, D = r.shape
    w = _finch_w(w, (B, H, D))
    st = _wkv5_state_arg("s", s, B, H, D)
    ls, sh = _launch_stream(r.device, stream)
    o = _out("o", o, (B, H, D), r.device, ls)
    _use_on(stream, st, r, k, v, w, u, o)
    status = lib.rwkv_wkv6_step(B, H, D, _ptr(st), _ptr(r), _ptr(k), _ptr(v), _ptr(w), _ptr(u),
                                _ptr(o), sh)
    _check("rwkv_wkv6_step", status)
    return o
