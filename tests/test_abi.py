"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status before
any HIP call.

Every call here is built to fail validation (or to be a zero-size no-op), so
no kernel is ever launched.  The fake device pointers are never dereferenced.
On a host with a GPU this module is skipped anyway: a validation bug there
would otherwise launch a kernel on fake pointers.
"""
import ctypes
import os
import re

import pytest

import linear_attention_sequence_rwkv_amd as rw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")

OK, NULLPTR, SHAPE, UNSUPPORTED, WORKSPACE, ALIGN, HIP = 0, -1, -2, -3, -4, -5, -6


def _declared_functions():
    names = set()
    for fn in os.listdir(HEADER_DIR):
        if fn.endswith(".h"):
            text = open(os.path.join(HEADER_DIR, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(rwkv_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rw.LIB_PATH):
        pytest.fail("librwkv_wkv.so is not built (run __graft_entry__.build())")
    return rw.load_library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert names == sorted([
        "rwkv_abi_version", "rwkv_status_str", "rwkv_last_hip_error",
        "rwkv_set_tuning", "rwkv_get_tuning", "rwkv_wkv4_workspace_error",
        "rwkv_wkv4_forward_workspace", "rwkv_wkv4_forward", "rwkv_wkv4_forward_state",
        "rwkv_wkv4_forward_noalloc",
        "rwkv_wkv4_backward_workspace", "rwkv_wkv4_backward",
        "rwkv_wkv4_forward_train", "rwkv_wkv4_backward_after_forward",
        "rwkv_wkv4_state_init", "rwkv_wkv4_step", "rwkv_wkv5_forward_workspace",
        "rwkv_wkv5_forward", "rwkv_wkv5_forward_state", "rwkv_wkv5_step",
        "rwkv_wkv6_forward_workspace", "rwkv_wkv6_forward", "rwkv_wkv6_step",
    ])


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert name in rw._SIGNATURES, name


def test_exports_nothing_else(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", rw.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert {n for n in exported if n.startswith("rwkv_")} == set(_declared_functions())


def test_version_and_status_strings(lib):
    assert lib.rwkv_abi_version() == 1
    for s in (OK, NULLPTR, SHAPE, UNSUPPORTED, WORKSPACE, ALIGN, HIP):
        assert lib.rwkv_status_str(s)
    assert lib.rwkv_status_str(12345) == b"unknown status"
    assert lib.rwkv_last_hip_error() == 0


def _skip_if_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("error-path checks run on hosts without a GPU only")


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10004)
NULL = ctypes.c_void_p(0)


def test_wkv4_forward_rejections(lib):
    _skip_if_gpu()
    f = lib.rwkv_wkv4_forward
    need = lib.rwkv_wkv4_forward_workspace(8, 1024, 768)
    assert need > 0
    args = lambda **kw: [kw.get(n, FAKE) for n in ("w", "u", "k", "v", "y")]  # noqa: E731
    # zero sizes are a no-op even with NULL pointers
    assert f(0, 1024, 768, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == OK
    assert f(8, 0, 768, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == OK
    assert f(8, 1024, 0, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == OK
    # negative and overflowing sizes
    assert f(-1, 1024, 768, *args(), FAKE, need, NULL) == SHAPE
    assert f(8, -5, 768, *args(), FAKE, need, NULL) == SHAPE
    assert f(1 << 40, 1 << 20, 1 << 20, *args(), FAKE, need, NULL) == SHAPE
    # each required pointer
    for n in ("w", "u", "k", "v", "y"):
        assert f(8, 1024, 768, *args(**{n: NULL}), FAKE, need, NULL) == NULLPTR, n
        assert f(8, 1024, 768, *args(**{n: MISALIGNED}), FAKE, need, NULL) == ALIGN, n
    # workspace
    assert f(8, 1024, 768, *args(), NULL, need, NULL) == WORKSPACE
    assert f(8, 1024, 768, *args(), FAKE, need - 1, NULL) == WORKSPACE
    assert f(8, 1024, 768, *args(), MISALIGNED, need, NULL) == ALIGN
    # too many tiles for 32-bit tickets
    assert f(1 << 24, 1 << 20, 64, *args(), FAKE, 1 << 62, NULL) == UNSUPPORTED
    assert lib.rwkv_last_hip_error() == 0


def test_wkv4_workspace_sizes(lib):
    assert lib.rwkv_wkv4_forward_workspace(0, 10, 10) == 0
    assert lib.rwkv_wkv4_forward_workspace(-1, 10, 10) == 0
    small = lib.rwkv_wkv4_forward_workspace(1, 64, 64)
    big = lib.rwkv_wkv4_forward_workspace(1, 65536, 5120)
    assert 0 < small < big
    # grows with the number of tiles and channel blocks
    assert lib.rwkv_wkv4_forward_workspace(2, 65536, 5120) > big


def test_wkv4_step_and_init_rejections(lib):
    _skip_if_gpu()
    s = lib.rwkv_wkv4_step
    ptrs = lambda **kw: [kw.get(n, FAKE) for n in "a b p w u k v y".split()]  # noqa: E731
    assert s(0, 4096, *[NULL] * 8, NULL) == OK
    assert s(-2, 4096, *ptrs(), NULL) == SHAPE
    for n in "a b p w u k v y".split():
        assert s(256, 4096, *ptrs(**{n: NULL}), NULL) == NULLPTR, n
        assert s(256, 4096, *ptrs(**{n: MISALIGNED}), NULL) == ALIGN, n
    i = lib.rwkv_wkv4_state_init
    assert i(0, 4, NULL, NULL, NULL, NULL) == OK
    assert i(4, -4, FAKE, FAKE, FAKE, NULL) == SHAPE
    assert i(4, 4, FAKE, NULL, FAKE, NULL) == NULLPTR
    assert i(4, 4, FAKE, FAKE, MISALIGNED, NULL) == ALIGN


def test_wkv5_rejections(lib):
    _skip_if_gpu()
    f = lib.rwkv_wkv5_forward
    ptrs = lambda **kw: [kw.get(n, FAKE) for n in "r k v w u o".split()]  # noqa: E731
    need = lib.rwkv_wkv5_forward_workspace(4, 4096, 32, 64)
    assert f(0, 4096, 32, 64, *[NULL] * 6, NULL, 0, NULL) == OK
    assert f(4, 4096, 32, 32, *ptrs(), FAKE, need, NULL) == UNSUPPORTED
    # chunks stream through 32-bit buffer ranges of 64 rows of H*D floats
    assert f(1, 64, 65536, 64, *ptrs(), FAKE, 1 << 40, NULL) == UNSUPPORTED
    assert f(4, -1, 32, 64, *ptrs(), FAKE, need, NULL) == SHAPE
    for n in "r k v w u o".split():
        assert f(4, 4096, 32, 64, *ptrs(**{n: NULL}), FAKE, need, NULL) == NULLPTR, n
        assert f(4, 4096, 32, 64, *ptrs(**{n: MISALIGNED}), FAKE, need, NULL) == ALIGN, n
    assert lib.rwkv_wkv5_forward_workspace(4, 4096, 32, 32) == 0


def test_wkv4_forward_state_rejections(lib):
    _skip_if_gpu()
    f = lib.rwkv_wkv4_forward_state
    need = lib.rwkv_wkv4_forward_workspace(2, 300, 128)
    names = "w u k v y a_in b_in p_in a_out b_out p_out".split()
    args = lambda **kw: [kw.get(n, FAKE) for n in names]  # noqa: E731
    assert f(0, 300, 128, *[NULL] * 11, NULL, 0, NULL) == OK
    assert f(2, -1, 128, *args(), FAKE, need, NULL) == SHAPE
    for n in names[:5]:
        assert f(2, 300, 128, *args(**{n: NULL}), FAKE, need, NULL) == NULLPTR, n
    # a state triple is all or nothing
    for n in names[5:]:
        assert f(2, 300, 128, *args(**{n: NULL}), FAKE, need, NULL) == NULLPTR, n
        assert f(2, 300, 128, *args(**{n: MISALIGNED}), FAKE, need, NULL) == ALIGN, n
    # both triples absent: the plain forward's checks
    none = dict(a_in=NULL, b_in=NULL, p_in=NULL, a_out=NULL, b_out=NULL, p_out=NULL)
    assert f(2, 300, 128, *args(**none), NULL, need, NULL) == WORKSPACE
    assert f(2, 300, 128, *args(**none, y=MISALIGNED), FAKE, need, NULL) == ALIGN
    assert lib.rwkv_last_hip_error() == 0


def test_wkv5_state_and_step_rejections(lib):
    _skip_if_gpu()
    f = lib.rwkv_wkv5_forward_state
    names = "r k v w u o s_in s_out".split()
    ptrs = lambda **kw: [kw.get(n, FAKE) for n in names]  # noqa: E731
    assert f(0, 64, 2, 64, *[NULL] * 8, NULL, 0, NULL) == OK
    assert f(1, 64, 2, 16, *ptrs(), NULL, 0, NULL) == UNSUPPORTED
    for n in names[:6]:
        assert f(1, 64, 2, 64, *ptrs(**{n: NULL}), NULL, 0, NULL) == NULLPTR, n
    for n in names:
        assert f(1, 64, 2, 64, *ptrs(**{n: MISALIGNED}), NULL, 0, NULL) == ALIGN, n
    s = lib.rwkv_wkv5_step
    names = "s r k v w u o".split()
    ptrs = lambda **kw: [kw.get(n, FAKE) for n in names]  # noqa: E731
    assert s(0, 2, 64, *[NULL] * 7, NULL) == OK
    assert s(1, 2, 32, *ptrs(), NULL) == UNSUPPORTED
    assert s(1, -2, 64, *ptrs(), NULL) == SHAPE
    for n in names:
        assert s(1, 2, 64, *ptrs(**{n: NULL}), NULL) == NULLPTR, n
        assert s(1, 2, 64, *ptrs(**{n: MISALIGNED}), NULL) == ALIGN, n
    assert lib.rwkv_last_hip_error() == 0


@pytest.mark.parametrize("entry", ["rwkv_wkv4_backward", "rwkv_wkv4_backward_after_forward"])
def test_wkv4_backward_rejections(lib, entry):
    _skip_if_gpu()
    f = getattr(lib, entry)
    need = lib.rwkv_wkv4_backward_workspace(2, 300, 128)
    assert need > lib.rwkv_wkv4_forward_workspace(2, 300, 128)
    names = "w u k v gy gw gu gk gv".split()
    args = lambda **kw: [kw.get(n, FAKE) for n in names]  # noqa: E731
    assert f(0, 300, 128, *[NULL] * 9, NULL, 0, NULL) == OK
    assert f(2, -1, 128, *args(), FAKE, need, NULL) == SHAPE
    for n in names:
        assert f(2, 300, 128, *args(**{n: NULL}), FAKE, need, NULL) == NULLPTR, n
        assert f(2, 300, 128, *args(**{n: MISALIGNED}), FAKE, need, NULL) == ALIGN, n
    assert f(2, 300, 128, *args(), NULL, need, NULL) == WORKSPACE
    assert f(2, 300, 128, *args(), FAKE, need - 1, NULL) == WORKSPACE
    assert f(2, 300, 128, *args(), MISALIGNED, need, NULL) == ALIGN
    assert lib.rwkv_wkv4_backward_workspace(0, 10, 10) == 0
    assert lib.rwkv_last_hip_error() == 0


def test_wkv4_forward_train_rejections(lib):
    """The training forward takes a backward workspace: a forward-sized one is
    rejected before anything is launched."""
    _skip_if_gpu()
    f = lib.rwkv_wkv4_forward_train
    need = lib.rwkv_wkv4_backward_workspace(2, 300, 128)
    small = lib.rwkv_wkv4_forward_workspace(2, 300, 128)
    names = "w u k v y".split()
    args = lambda **kw: [kw.get(n, FAKE) for n in names]  # noqa: E731
    assert f(0, 300, 128, *[NULL] * 5, NULL, 0, NULL) == OK
    assert f(2, -1, 128, *args(), FAKE, need, NULL) == SHAPE
    for n in names:
        assert f(2, 300, 128, *args(**{n: NULL}), FAKE, need, NULL) == NULLPTR, n
        assert f(2, 300, 128, *args(**{n: MISALIGNED}), FAKE, need, NULL) == ALIGN, n
    assert f(2, 300, 128, *args(), NULL, need, NULL) == WORKSPACE
    assert f(2, 300, 128, *args(), FAKE, small, NULL) == WORKSPACE
    assert f(2, 300, 128, *args(), FAKE, need - 1, NULL) == WORKSPACE
    assert f(2, 300, 128, *args(), MISALIGNED, need, NULL) == ALIGN
    assert lib.rwkv_last_hip_error() == 0


def test_wkv6_rejections(lib):
    _skip_if_gpu()
    f = lib.rwkv_wkv6_forward
    names = "r k v w u o s_in s_out".split()
    ptrs = lambda **kw: [kw.get(n, FAKE) for n in names]  # noqa: E731
    need = lib.rwkv_wkv6_forward_workspace(4, 4096, 32, 64)
    assert need > 0 and lib.rwkv_wkv6_forward_workspace(4, 4096, 32, 32) == 0
    assert f(0, 64, 2, 64, *[NULL] * 8, NULL, 0, NULL) == OK
    assert f(1, 64, 2, 32, *ptrs(), NULL, 0, NULL) == UNSUPPORTED
    assert f(1, 64, 65536, 64, *ptrs(), FAKE, 1 << 40, NULL) == UNSUPPORTED
    assert f(1, -64, 2, 64, *ptrs(), NULL, 0, NULL) == SHAPE
    for n in names[:6]:
        assert f(1, 64, 2, 64, *ptrs(**{n: NULL}), NULL, 0, NULL) == NULLPTR, n
    for n in names:
        assert f(1, 64, 2, 64, *ptrs(**{n: MISALIGNED}), NULL, 0, NULL) == ALIGN, n
    assert f(4, 4096, 32, 64, *ptrs(), NULL, need, NULL) == WORKSPACE
    assert f(4, 4096, 32, 64, *ptrs(), FAKE, need - 1, NULL) == WORKSPACE
    st = lib.rwkv_wkv6_step
    names = "s r k v w u o".split()
    ptrs = lambda **kw: [kw.get(n, FAKE) for n in names]  # noqa: E731
    assert st(0, 2, 64, *[NULL] * 7, NULL) == OK
    assert st(1, 2, 16, *ptrs(), NULL) == UNSUPPORTED
    for n in names:
        assert st(1, 2, 64, *ptrs(**{n: NULL}), NULL) == NULLPTR, n
        assert st(1, 2, 64, *ptrs(**{n: MISALIGNED}), NULL) == ALIGN, n
    assert lib.rwkv_last_hip_error() == 0


def test_tuning_overrides(lib):
    """Plan overrides: unknown keys and values are rejected, accepted ones are
    read back, and they change the plan (hence the workspace sizes)."""
    keys = (1, 2, 3, 4, 5, 6, 7)
    old = {k: lib.rwkv_get_tuning(k) for k in keys}
    try:
        assert lib.rwkv_set_tuning(0, 1) == UNSUPPORTED
        assert lib.rwkv_set_tuning(8, 1) == UNSUPPORTED
        assert lib.rwkv_set_tuning(7, -1) == UNSUPPORTED
        assert lib.rwkv_set_tuning(1, 13205) == UNSUPPORTED   # no such tile shape
        assert lib.rwkv_set_tuning(1, 1) == UNSUPPORTED       # cpl 0: once a SIGFPE
        assert lib.rwkv_set_tuning(2, 2) == UNSUPPORTED
        assert lib.rwkv_set_tuning(3, 48) == UNSUPPORTED
        assert lib.rwkv_set_tuning(5, 16) == UNSUPPORTED
        assert lib.rwkv_set_tuning(4, -1) == UNSUPPORTED
        for key, val in ((1, 40808), (2, 1), (3, 16), (4, 2), (5, 32), (6, 3), (7, 1)):
            assert lib.rwkv_set_tuning(key, val) == OK
            assert lib.rwkv_get_tuning(key) == val
        # the Eagle workspace holds one state per head and earlier segment
        assert lib.rwkv_set_tuning(4, 1) == OK
        assert lib.rwkv_wkv5_forward_workspace(4, 4096, 32, 64) == 0
        assert lib.rwkv_set_tuning(4, 4) == OK
        assert lib.rwkv_wkv5_forward_workspace(4, 4096, 32, 64) == 4 * 32 * 3 * 64 * 64 * 4
        # a 4-channel tile shape does not apply where 4 does not divide C
        a = lib.rwkv_wkv4_forward_workspace(1, 1000, 66)
        assert lib.rwkv_set_tuning(1, 0) == OK
        assert lib.rwkv_wkv4_forward_workspace(1, 1000, 66) == a
    finally:
        for k, v in old.items():
            assert lib.rwkv_set_tuning(k, v) == OK


def test_wkv4_sequence_length_limit(lib):
    """Decay counts are float32 integers: one call takes T <= 2^24 - 64."""
    limit = (1 << 24) - 64
    assert lib.rwkv_wkv4_forward_workspace(1, limit, 64) > 0
    assert lib.rwkv_wkv4_forward_workspace(1, limit + 1, 64) == 0
    assert lib.rwkv_wkv4_backward_workspace(1, limit, 64) > 0
    assert lib.rwkv_wkv4_backward_workspace(1, limit + 1, 64) == 0
    _skip_if_gpu()
    args = [FAKE] * 5
    assert lib.rwkv_wkv4_forward(1, limit + 1, 64, *args, FAKE, 1 << 62, NULL) == UNSUPPORTED
    assert lib.rwkv_wkv4_forward_state(1, limit + 1, 64, *args, *[NULL] * 6, FAKE, 1 << 62,
                                       NULL) == UNSUPPORTED
    assert lib.rwkv_wkv4_backward(1, limit + 1, 64, *[FAKE] * 9, FAKE, 1 << 62,
                                  NULL) == UNSUPPORTED
    assert lib.rwkv_wkv4_forward_train(1, limit + 1, 64, *args, FAKE, 1 << 62,
                                       NULL) == UNSUPPORTED
    assert lib.rwkv_last_hip_error() == 0


def test_workspace_error_query_rejections(lib):
    _skip_if_gpu()
    q = lib.rwkv_wkv4_workspace_error
    assert q(NULL, 256, FAKE, NULL) == NULLPTR
    assert q(FAKE, 256, NULL, NULL) == NULLPTR
    assert q(FAKE, 3, FAKE, NULL) == WORKSPACE
    assert q(MISALIGNED, 256, FAKE, NULL) == ALIGN
    assert lib.rwkv_last_hip_error() == 0


def test_wkv4_forward_noalloc_rejections(lib):
    """The no-allocation forward checks what the plain forward checks, and
    rejects shapes whose workspace exceeds its 32 MiB array, before any HIP
    call."""
    _skip_if_gpu()
    f = lib.rwkv_wkv4_forward_noalloc
    args = lambda **kw: [kw.get(n, FAKE) for n in ("w", "u", "k", "v", "y")]  # noqa: E731
    assert f(0, 1024, 768, NULL, NULL, NULL, NULL, NULL, NULL) == OK
    assert f(-1, 1024, 768, *args(), NULL) == SHAPE
    for n in ("w", "u", "k", "v", "y"):
        assert f(8, 1024, 768, *args(**{n: NULL}), NULL) == NULLPTR, n
        assert f(8, 1024, 768, *args(**{n: MISALIGNED}), NULL) == ALIGN, n
    assert lib.rwkv_wkv4_forward_workspace(1, 65536, 5120) > 32 << 20
    assert f(1, 65536, 5120, *args(), NULL) == WORKSPACE
    assert f(1, (1 << 24) - 63, 64, *args(), NULL) == UNSUPPORTED
    assert lib.rwkv_last_hip_error() == 0
