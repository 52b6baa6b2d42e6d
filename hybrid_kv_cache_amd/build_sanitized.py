"""Host-sanitizer build of libfkv: the C ABI layer (api.cpp: argument checks,
plans, offsets, the classification and rolling-mask helpers) compiled with
AddressSanitizer and UndefinedBehaviorSanitizer by g++, linked with the
ordinary gfx950 kernel objects of hybrid_kv_cache_amd/_build (device code is
never built with a sanitizer).

    python -m hybrid_kv_cache_amd.build_sanitized      # prints the library path

Running Python code against it needs the ASan runtime preloaded and the
binding pointed at it (sanitized_env() gives the variables):
    FKV_LIB=<path> LD_PRELOAD=<libasan.so> ASAN_OPTIONS=detect_leaks=0 ...
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

from hybrid_kv_cache_amd import build as _build

PKG = _build.PKG
SAN_DIR = os.path.join(_build.OUT_DIR, "sanitized")
SAN_LIB = os.path.join(SAN_DIR, "libfkv_san.so")
KERNEL_SOURCES = [s for s in _build.SOURCES if s.endswith(".hip")]
ROCM = "/opt/rocm"


def gxx() -> str:
    path = shutil.which("g++")
    if not path:
        raise RuntimeError("g++ not found: the host-sanitizer build needs it")
    return path


def asan_runtime() -> str:
    """The ASan runtime matching g++ (to be preloaded into the interpreter)."""
    r = subprocess.run([gxx(), "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("libasan.so of g++ not found")
    return path


def build(verbose: bool = False) -> str:
    """Compile api.cpp with -fsanitize=address,undefined and link it with the
    kernel objects (building those first if they are missing)."""
    objs = [os.path.join(_build.OUT_DIR, os.path.splitext(s)[0] + ".o") for s in KERNEL_SOURCES]
    if not all(os.path.exists(o) for o in objs):
        _build.build()
    os.makedirs(SAN_DIR, exist_ok=True)
    api_o = os.path.join(SAN_DIR, "api_san.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]
    cmd = [gxx(), "-std=c++17", "-O1", "-g", "-fPIC", "-Wall", "-Wno-unused-result"] + san + [
        "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
        f"-I{os.path.join(_build.ROOT, 'include')}", f"-I{_build.CSRC}",
        "-c", os.path.join(_build.CSRC, "api.cpp"), "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    tmp = SAN_LIB + ".tmp"
    cmd = [gxx(), "-shared"] + san + ["-o", tmp, api_o] + objs + [
        f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(SAN_LIB)
    return SAN_LIB


def sanitized_env(base=None) -> dict:
    """Environment for a Python process that loads the sanitized library
    through the binding: errors abort the process with a report."""
    env = dict(os.environ if base is None else base)
    env["FKV_LIB"] = SAN_LIB
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
