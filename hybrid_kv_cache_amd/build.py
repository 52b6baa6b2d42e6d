"""Build libfkv.so in-tree with hipcc for gfx950.

    python -m hybrid_kv_cache_amd.build          # or __graft_entry__.build()

Every source is compiled each time (the build is the "does it compile"
check); objects go to hybrid_kv_cache_amd/_build/, the library to
hybrid_kv_cache_amd/libfkv.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfkv.so")
SOURCES = ["api.cpp", "score.hip", "select.hip", "compact.hip", "attend.hip", "tokens.hip", "attend_fp8.hip", "calib.hip", "scratch.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfkv.so)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
            "-Wall", "-Wno-unused-result"]


def device_flags():
    # Keep the compiler from forming packed fp32 (v_pk_*_f32) instructions.
    return ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-ffp-contract=fast", "-munsafe-fp-atomics"]


# Kernels whose inputs are finite by contract (masked scores are -inf, never
# NaN): fmax needs no NaN quieting there.
NO_NAN_SOURCES = {"attend.hip", "score.hip"}


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags()
    if src.endswith(".hip"):
        cmd += device_flags() + ["-x", "hip"]
        if src in NO_NAN_SOURCES:
            cmd += ["-fno-honor-nans"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
