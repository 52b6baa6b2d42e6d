"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: the ABI tests (argument checks, plans, offsets,
the rolling-mask and head-classification helpers, all on the CPU) run again
in a child interpreter against libfkv built with -fsanitize=address,undefined
for its host code; any report aborts the child and fails this test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is needed for the sanitizer build")
def test_abi_tests_clean_under_asan_ubsan():
    from hybrid_kv_cache_amd import build_sanitized as S
    lib = S.build()
    # the library is instrumented (calls into both runtimes)
    undef = subprocess.run(["nm", "-u", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in undef and "__ubsan_handle" in undef
    env = S.sanitized_env()
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py"),
           os.path.join(ROOT, "tests", "test_oracle_profile.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    # the child really loaded the sanitized build
    probe = subprocess.run([sys.executable, "-c",
                            "from hybrid_kv_cache_amd import fkv; fkv.load(); print(fkv.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stdout + probe.stderr
