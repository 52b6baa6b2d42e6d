"""Host check of the attention kernels' work schedules (no GPU).

Builds tests/sched_cover.cpp host-only with hipcc: it calls the library's own
schedule decoder (the per-workgroup work assignment of the bf16 and fp8
attention kernels, from fkv_device.h) for every workgroup of many launches
(1 .. 5 rounds of pairs, 8 to 304 CUs, uniform, ragged and empty heads, with
and without a partial-result buffer) and checks that every key tile of every
(head, query tile) pair is computed exactly once, that the parts of every cut
pair write the partial-result slots the combine kernel merges, and that no
two pairs share a slot.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "hybrid_kv_cache_amd", "csrc")


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_every_tile_once_and_slots_match_the_combine(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "sched_cover")
    subprocess.run([hipcc, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1",
                    "-I", CSRC, os.path.join(HERE, "sched_cover.cpp"), "-o", exe],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:]
    assert r.stdout.startswith("OK"), r.stdout
