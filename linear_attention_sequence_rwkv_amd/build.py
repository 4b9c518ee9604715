"""Build librwkv_wkv.so (HIP for gfx950) in-tree.

    python -m linear_attention_sequence_rwkv_amd.build

Each source under csrc/ is compiled by hipcc into _build/ in parallel and
linked into linear_attention_sequence_rwkv_amd/librwkv_wkv.so.  The
benchmark's copy-peak kernel (benchsrc/copy_peak.hip) becomes a library of
its own, libwkv_copy_peak.so, next to it.  Every call recompiles (the build
is a few seconds per file).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "librwkv_wkv.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
COPY_PEAK_SRC = os.path.join(PKG, "benchsrc", "copy_peak.hip")
COPY_PEAK_PATH = os.path.join(PKG, "libwkv_copy_peak.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 VALU forms in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build the WKV library")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(hipcc: str, src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags or [])
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, extra), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    _link_one(hipcc, _compile(hipcc, COPY_PEAK_SRC, extra), COPY_PEAK_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources, and {COPY_PEAK_PATH}")
    return LIB_PATH


def _link_one(hipcc: str, obj: str, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
