"""C-ABI contract of libfkv.so on the host (no GPU needed).

Loads the built library, checks that every function include/fkv.h declares
is exported, and drives the argument checks and the host-side plan, all of
which return before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from hybrid_kv_cache_amd import fkv
from hybrid_kv_cache_amd import workloads as W
from oracle import forcing_kv as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fkv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fkv.LIB_PATH):
        pytest.fail("libfkv.so is not built: run python -m hybrid_kv_cache_amd.build")
    return fkv.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fkv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(fkv.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fkv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(fkv.FkvDesc) == 32
    assert ctypes.sizeof(fkv.FkvCkv) == 56


def test_status_strings(lib):
    for st in range(8):
        assert fkv.fkv_status_str(st)
    assert fkv.fkv_status_str(99) == "unknown status"


def _plan(desc, role, mask, m):
    lib = fkv.load()
    kept = ctypes.c_int64(-1)
    ws = ctypes.c_size_t(0)
    role = np.ascontiguousarray(role, np.uint8)
    mask = np.ascontiguousarray(mask, np.uint8)
    st = lib.fkv_plan(ctypes.byref(desc) if desc is not None else None, role.ctypes.data,
                      mask.ctypes.data if mask.size else None, m, ctypes.byref(kept),
                      ctypes.byref(ws))
    return st, kept.value, ws.value


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_plan_matches_oracle_offsets(lib, name):
    w = W.WORKLOADS[name]
    rng = np.random.default_rng(1)
    role = np.zeros(w.num_heads, np.uint8)
    role[rng.permutation(w.num_heads)[: w.num_heads - w.num_static]] = 1
    mask = np.tile(W.chunk_boundary_mask(w.hist_frames), (w.num_heads, 1))
    st, kept_tokens, ws = _plan(fkv.desc_for(w), role, mask, w.budget_m)
    assert st == fkv.FKV_OK, fkv.fkv_last_error()
    kept = O.select_frames(np.zeros((w.num_heads, w.hist_frames)), role, mask, w.budget_m)
    _, _, tok_off = O.offsets(kept, w.tokens_per_frame, w.cur_frames)
    assert kept_tokens == tok_off[-1]
    n_dyn = int(role.sum())
    assert ws >= n_dyn * w.n_sampled * w.frames * 4


def test_plan_examples(lib):
    # the 480P layer: 6 static heads keep 12 frames, 6 dynamic keep 13
    d = fkv.make_desc(12, 128, 1560, 18, 3, 16)
    role = np.array([0] * 6 + [1] * 6, np.uint8)
    mask = np.tile(W.chunk_boundary_mask(18), (12, 1))
    st, kept, _ = _plan(d, role, mask, 13)
    assert st == 0 and kept == 6 * 15 * 1560 + 6 * 16 * 1560 == 290160
    # budget above the history keeps everything
    st, kept, _ = _plan(d, np.ones(12, np.uint8), mask, 100)
    assert st == 0 and kept == 12 * 21 * 1560


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 7, fkv.FKV_ERR_DTYPE),
    ("head_dim", 64, fkv.FKV_ERR_DTYPE),        # bf16 needs 128
    ("num_heads", 0, fkv.FKV_ERR_SHAPE),
    ("num_heads", 65, fkv.FKV_ERR_SHAPE),
    ("hist_frames", -1, fkv.FKV_ERR_SHAPE),
    ("hist_frames", 65, fkv.FKV_ERR_SHAPE),
    ("cur_frames", 0, fkv.FKV_ERR_SHAPE),
    ("tokens_per_frame", 0, fkv.FKV_ERR_SHAPE),
    ("query_stride", 0, fkv.FKV_ERR_SHAPE),
    ("scale", -1.0, fkv.FKV_ERR_SHAPE),
    ("tokens_per_frame", 1 << 19, fkv.FKV_ERR_SHAPE),   # 4 GiB window tensor
])
def test_plan_rejects_bad_desc(lib, field, value, status):
    d = fkv.make_desc(4, 128, 16, 6, 3, 4)
    setattr(d, field, value)
    st, _, _ = _plan(d, np.ones(max(d.num_heads, 1), np.uint8)[: max(d.num_heads, 1)],
                     np.ones((max(d.num_heads, 1), max(d.hist_frames, 0)), np.uint8), 2)
    assert st == status
    assert fkv.fkv_last_error()


def test_window_size_limit_edge(lib):
    """4 GiB is the first window-tensor size refused; one token-row less fits."""
    # 4 heads x 128 dims x 2 bytes = 1 KiB per token row, 9 frames per window
    rows_4g = (1 << 32) // 1024
    d = fkv.make_desc(4, 128, rows_4g // 9 + 1, 6, 3, 4)
    st, _, _ = _plan(d, np.ones(4, np.uint8), np.zeros((4, 6), np.uint8), 2)
    assert st == fkv.FKV_ERR_SHAPE and "4 GiB" in fkv.fkv_last_error()
    d = fkv.make_desc(4, 128, (rows_4g - 1) // 9, 6, 3, 4)
    st, _, _ = _plan(d, np.ones(4, np.uint8), np.zeros((4, 6), np.uint8), 2)
    assert st == fkv.FKV_OK


def test_plan_null_and_budget(lib):
    d = fkv.make_desc(2, 128, 16, 4, 3, 4)
    st, _, _ = _plan(None, np.ones(2, np.uint8), np.ones((2, 4), np.uint8), 2)
    assert st == fkv.FKV_ERR_NULL
    st, _, _ = _plan(d, np.ones(2, np.uint8), np.ones((2, 4), np.uint8), -1)
    assert st == fkv.FKV_ERR_BUDGET
    st, _, _ = _plan(d, np.array([1, 2], np.uint8), np.ones((2, 4), np.uint8), 2)
    assert st == fkv.FKV_ERR_SHAPE
    # static heads without a mask
    lib = fkv.load()
    role = np.zeros(2, np.uint8)
    st = lib.fkv_plan(ctypes.byref(d), role.ctypes.data, None, 2, None, None)
    assert st == fkv.FKV_ERR_NULL
    # all dynamic: the mask may be NULL
    role = np.ones(2, np.uint8)
    st = lib.fkv_plan(ctypes.byref(d), role.ctypes.data, None, 2, None, None)
    assert st == fkv.FKV_OK


def _compress_status(d, cap, ws_bytes, null_k=False, null_ws=False):
    lib = fkv.load()
    role = np.ones(d.num_heads, np.uint8)
    mask = np.zeros((d.num_heads, d.hist_frames), np.uint8)
    fake = 0x1000  # never dereferenced: every check below fails before HIP
    ckv = fkv.FkvCkv(None if null_k else fake, fake, fake, fake, fake, None, cap)
    return lib.fkv_compress(ctypes.byref(d), fake, fake, fake, role.ctypes.data,
                            mask.ctypes.data, 2, ctypes.byref(ckv),
                            None if null_ws else fake, ws_bytes, None)


def test_compress_argument_errors_before_any_hip_call(lib):
    d = fkv.make_desc(2, 128, 16, 4, 3, 4)
    st, kept, ws = _plan(d, np.ones(2, np.uint8), np.zeros((2, 4), np.uint8), 2)
    assert st == 0
    assert _compress_status(d, kept - 1, ws) == fkv.FKV_ERR_CAPACITY
    assert _compress_status(d, kept, ws - 1) == fkv.FKV_ERR_WORKSPACE
    assert _compress_status(d, kept, ws, null_ws=True) == fkv.FKV_ERR_WORKSPACE
    assert _compress_status(d, kept, ws, null_k=True) == fkv.FKV_ERR_NULL
    assert "cap_tokens" in _capture_error(d, kept - 1, ws)


def test_compress_attend_argument_errors_before_any_hip_call(lib):
    """The combined compression and attention call checks the attention
    output and the compression arguments on the host, like fkv_compress."""
    d = fkv.make_desc(2, 128, 16, 4, 3, 4)
    role, mask = np.ones(2, np.uint8), np.zeros((2, 4), np.uint8)
    st, kept, ws = _plan(d, role, mask, 2)
    assert st == 0
    fake = ctypes.c_void_p(0x1000)

    def call(cap, ws_bytes, out=fake):
        ckv = fkv.FkvCkv(fake, fake, fake, fake, fake, None, cap)
        return lib.fkv_compress_attend(ctypes.byref(d), fake, fake, fake, role.ctypes.data,
                                       mask.ctypes.data, 2, ctypes.byref(ckv), fake, ws_bytes,
                                       out, None, 0, None)

    assert call(kept, ws, out=None) == fkv.FKV_ERR_NULL
    assert "attend_out" in fkv.fkv_last_error()
    assert call(kept - 1, ws) == fkv.FKV_ERR_CAPACITY
    assert call(kept, ws - 1) == fkv.FKV_ERR_WORKSPACE


def test_compress_noalloc_argument_errors_before_any_hip_call(lib):
    """The allocation-free entry point checks its arguments and its scratch
    limit on the host: a layer whose workspace exceeds the library's scratch
    size is refused with a message naming both sizes."""
    d = fkv.make_desc(2, 128, 16, 4, 3, 4)
    role, mask = np.ones(2, np.uint8), np.zeros((2, 4), np.uint8)
    st, kept, ws = _plan(d, role, mask, 2)
    assert st == 0 and ws <= fkv.SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)

    def call(desc, cap, q=fake, role=role, mask=mask, budget=2):
        ckv = fkv.FkvCkv(fake, fake, fake, fake, fake, None, cap)
        r = np.ascontiguousarray(role, np.uint8)
        m = np.ascontiguousarray(mask, np.uint8)
        return lib.fkv_compress_noalloc(ctypes.byref(desc), q, fake, fake, r.ctypes.data,
                                        m.ctypes.data, budget, ctypes.byref(ckv), None)

    assert call(d, kept - 1) == fkv.FKV_ERR_CAPACITY
    assert call(d, kept, q=None) == fkv.FKV_ERR_NULL
    assert lib.fkv_compress_noalloc(None, fake, fake, fake, None, None, 2, None,
                                    None) == fkv.FKV_ERR_NULL
    # 64 dynamic heads, T = 8160, every query scored: the per-query frame
    # sums alone need 64 * 24480 * 21 * 4 bytes, far beyond the scratch size
    big = fkv.make_desc(64, 128, 8160, 18, 3, 1)
    st, kept_big, ws_big = _plan(big, np.ones(64, np.uint8), np.zeros((64, 18), np.uint8), 12)
    assert st == 0 and ws_big > fkv.SCRATCH_BYTES
    assert call(big, kept_big, role=np.ones(64, np.uint8), mask=np.zeros((64, 18), np.uint8),
                budget=12) == fkv.FKV_ERR_WORKSPACE
    msg = fkv.fkv_last_error()
    assert str(ws_big) in msg and str(fkv.SCRATCH_BYTES) in msg


def _capture_error(d, cap, ws):
    _compress_status(d, cap, ws)
    return fkv.fkv_last_error()


def test_attend_argument_errors(lib):
    d = fkv.make_desc(2, 128, 16, 4, 3, 4)
    ckv = fkv.FkvCkv(None, None, None, None, None, None, 0)
    assert lib.fkv_attend(ctypes.byref(d), 0x1000, ctypes.byref(ckv), 0x1000, None, 0,
                          None) == fkv.FKV_ERR_NULL
    assert lib.fkv_attend_dense(ctypes.byref(d), 0x1000, None, 0x1000, 0x1000, None, 0,
                                None) == fkv.FKV_ERR_NULL
    d.dtype = 5
    assert lib.fkv_attend_dense(ctypes.byref(d), 1, 1, 1, 1, None, 0, None) == fkv.FKV_ERR_DTYPE


def test_attend_fp8_argument_errors(lib):
    """fkv_attend_fp8 rejects, on the host: a missing cache or query, missing
    or non-positive scales, and a non-bf16 descriptor."""
    import numpy as np
    d = fkv.make_desc(2, 128, 16, 4, 3, 4)
    good = np.ones(3 * 2, dtype=np.float32)
    ckv = fkv.FkvCkv(None, None, None, None, None, None, 0)
    assert lib.fkv_attend_fp8(ctypes.byref(d), 0x1000, ctypes.byref(ckv), good.ctypes.data,
                              0x1000, None, 0, None) == fkv.FKV_ERR_NULL
    full = fkv.FkvCkv(0x1000, 0x1000, 0x1000, None, None, None, 0)
    assert lib.fkv_attend_fp8(ctypes.byref(d), None, ctypes.byref(full), good.ctypes.data,
                              0x1000, None, 0, None) == fkv.FKV_ERR_NULL
    assert lib.fkv_attend_fp8(ctypes.byref(d), 0x1000, ctypes.byref(full), None, 0x1000, None,
                              0, None) != fkv.FKV_OK
    bad = good.copy()
    bad[4] = 0.0
    assert lib.fkv_attend_fp8(ctypes.byref(d), 0x1000, ctypes.byref(full), bad.ctypes.data,
                              0x1000, None, 0, None) != fkv.FKV_OK
    d32 = fkv.make_desc(2, 128, 16, 4, 3, 4, dtype="f32")
    assert lib.fkv_attend_fp8(ctypes.byref(d32), 0x1000, ctypes.byref(full), good.ctypes.data,
                              0x1000, None, 0, None) == fkv.FKV_ERR_DTYPE



def test_compress_fp8_timed_and_profile_argument_errors(lib):
    """The remaining entry points reject bad arguments on the host:
    fkv_compress_fp8 (plan errors first, then missing, zero or non-finite
    scales, a non-bf16 descriptor, missing inputs), fkv_compress_timed (missing
    inputs or time array), fkv_profile_workspace (NULL output; its size is
    H x n_s x (F_h + F_c) fp32 values) and fkv_profile_heads (missing buffers,
    a workspace below that size)."""
    d = fkv.make_desc(2, 128, 16, 4, 3, 4)
    role = np.array([0, 1], np.uint8)
    mask = np.ones((2, 4), np.uint8)
    r, m = role.ctypes.data, mask.ctypes.data
    ckv = fkv.FkvCkv(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0)
    good = np.ones(2 * 2, dtype=np.float32)
    x = 0x1000

    def fp8(desc=d, q=x, m_budget=2, scales=good.ctypes.data):
        return lib.fkv_compress_fp8(ctypes.byref(desc), q, x, x, r, m, m_budget, scales,
                                    ctypes.byref(ckv), None, 0, None)
    assert fp8(m_budget=-1) == fkv.FKV_ERR_BUDGET
    assert fp8(scales=None) == fkv.FKV_ERR_NULL
    for v in (0.0, -1.0, np.inf, np.nan):
        bad = good.copy()
        bad[3] = v
        assert fp8(scales=bad.ctypes.data) == fkv.FKV_ERR_SHAPE
        assert "kv_scales[3]" in fkv.fkv_last_error()
    assert fp8(desc=fkv.make_desc(2, 128, 16, 4, 3, 4, dtype="f32")) == fkv.FKV_ERR_DTYPE
    assert fp8(q=None) == fkv.FKV_ERR_NULL

    ms = (ctypes.c_float * 3)()
    assert lib.fkv_compress_timed(ctypes.byref(d), x, x, x, r, m, 2, ctypes.byref(ckv), None,
                                  0, None, None) == fkv.FKV_ERR_NULL
    assert lib.fkv_compress_timed(ctypes.byref(d), None, x, x, r, m, 2, ctypes.byref(ckv), None,
                                  0, None, ms) == fkv.FKV_ERR_NULL
    assert lib.fkv_compress_timed(ctypes.byref(d), x, x, x, r, m, -3, ctypes.byref(ckv), None,
                                  0, None, ms) == fkv.FKV_ERR_BUDGET

    n = ctypes.c_size_t(0)
    assert lib.fkv_profile_workspace(ctypes.byref(d), None) == fkv.FKV_ERR_NULL
    assert lib.fkv_profile_workspace(ctypes.byref(d), ctypes.byref(n)) == fkv.FKV_OK
    n_s = -(-3 * 16 // 4)
    assert n.value == 2 * n_s * (4 + 3) * 4
    assert lib.fkv_profile_heads(ctypes.byref(d), x, x, None, x, n.value,
                                 None) == fkv.FKV_ERR_NULL
    assert lib.fkv_profile_heads(ctypes.byref(d), x, x, x, x, n.value - 4,
                                 None) == fkv.FKV_ERR_WORKSPACE
    assert lib.fkv_profile_heads(ctypes.byref(d), x, x, x, None, n.value,
                                 None) == fkv.FKV_ERR_WORKSPACE
    d.query_stride = 0
    assert lib.fkv_profile_workspace(ctypes.byref(d), ctypes.byref(n)) == fkv.FKV_ERR_SHAPE


def test_misaligned_tensors_are_rejected(lib):
    """Every entry point refuses a tensor or workspace that does not start on
    a 16-byte boundary (the kernels move 16-byte pieces), on the host, before
    any HIP call: FKV_ERR_SHAPE with the text naming the argument group."""
    d = fkv.make_desc(2, 128, 16, 4, 3, 4)
    role = np.array([0, 1], np.uint8)
    mask = np.ones((2, 4), np.uint8)
    r, m = role.ctypes.data, mask.ctypes.data
    A, X = 0x1000, 0x1008    # aligned, misaligned by 8 bytes
    ckv = fkv.FkvCkv(A, A, A, A, A, A, 1 << 20)
    bad_k = fkv.FkvCkv(X, A, A, A, A, A, 1 << 20)
    scales = np.ones(3 * 2, np.float32)
    cfg = fkv.FkvTokenCfg(1, 1, 8, 2)
    hist_frames = np.array([4, 4], np.int32)
    calls = [
        lambda: lib.fkv_compress(ctypes.byref(d), X, A, A, r, m, 2, ctypes.byref(ckv), A, 1 << 20,
                                 None),
        lambda: lib.fkv_compress(ctypes.byref(d), A, A, A, r, m, 2, ctypes.byref(bad_k), A,
                                 1 << 20, None),
        lambda: lib.fkv_compress(ctypes.byref(d), A, A, A, r, m, 2, ctypes.byref(ckv), X,
                                 1 << 20, None),
        lambda: lib.fkv_compress_noalloc(ctypes.byref(d), A, A, X, r, m, 2, ctypes.byref(ckv),
                                         None),
        lambda: lib.fkv_compress_attend(ctypes.byref(d), A, A, A, r, m, 2, ctypes.byref(ckv), A,
                                        1 << 20, X, None, 0, None),
        lambda: lib.fkv_compress_fp8(ctypes.byref(d), A, X, A, r, m, 2, scales.ctypes.data,
                                     ctypes.byref(ckv), A, 1 << 20, None),
        lambda: lib.fkv_compress_ragged(ctypes.byref(d), A, ctypes.byref(ckv),
                                        hist_frames.ctypes.data, X, A, r, m, 2,
                                        ctypes.byref(fkv.FkvCkv(A + 16, A + 16, A + 16, A + 16,
                                                                A + 16, A + 16, 1 << 20)),
                                        A, 1 << 20, None),
        lambda: lib.fkv_refresh_current(ctypes.byref(d), A, X, ctypes.byref(ckv), None),
        lambda: lib.fkv_compress_tokens(ctypes.byref(d), ctypes.byref(cfg), A, X, A, r,
                                        ctypes.byref(ckv), None, A, 1 << 20, None),
        lambda: lib.fkv_attend(ctypes.byref(d), X, ctypes.byref(ckv), A, None, 0, None),
        lambda: lib.fkv_attend(ctypes.byref(d), A, ctypes.byref(ckv), A, X, 1 << 30, None),
        lambda: lib.fkv_attend_dense(ctypes.byref(d), A, A, X, A, None, 0, None),
        lambda: lib.fkv_attend_fp8(ctypes.byref(d), A, ctypes.byref(ckv), scales.ctypes.data, X,
                                   None, 0, None),
        lambda: lib.fkv_profile_heads(ctypes.byref(d), A, A, A, X, 1 << 20, None),
    ]
    for i, call in enumerate(calls):
        assert call() == fkv.FKV_ERR_SHAPE, (i, fkv.fkv_last_error())
        assert "16-byte aligned" in fkv.fkv_last_error(), (i, fkv.fkv_last_error())

def test_attend_workspace_query(lib):
    """The workspace figure: NULL output rejected, bad descriptors rejected,
    0 for fp32 (no balanced schedule there), and for bf16 either a positive
    figure (a device is visible) or FKV_ERR_HIP (none is)."""
    d = fkv.make_desc(2, 128, 16, 4, 3, 4)
    assert lib.fkv_attend_workspace(ctypes.byref(d), None) == fkv.FKV_ERR_NULL
    n = ctypes.c_size_t(123)
    st = lib.fkv_attend_workspace(ctypes.byref(d), ctypes.byref(n))
    assert (st == fkv.FKV_OK and n.value > 0) or (st == fkv.FKV_ERR_HIP and n.value == 0)
    f = fkv.make_desc(2, 64, 16, 4, 3, 4, dtype="f32")
    n = ctypes.c_size_t(123)
    assert lib.fkv_attend_workspace(ctypes.byref(f), ctypes.byref(n)) == fkv.FKV_OK
    assert n.value == 0
    d.head_dim = 96
    assert lib.fkv_attend_workspace(ctypes.byref(d), ctypes.byref(n)) == fkv.FKV_ERR_DTYPE


# ---- rolling cache: host logic ---------------------------------------------

def test_roll_static_mask_matches_oracle(lib):
    """The library's keep rule for static heads in a rolling cache against the
    oracle's, on random histories (sorted distinct ids, with and without the
    sink) and caps."""
    rng = np.random.default_rng(0)
    for _ in range(400):
        fc = int(rng.integers(1, 6))
        n = int(rng.integers(0, 40))
        ids = sorted(rng.choice(200, n, replace=False).tolist())
        if n and rng.random() < 0.5:
            ids[0] = 0
            ids = sorted(set(ids))
        cap = int(rng.integers(0, 20))
        got = fkv.fkv_roll_static_mask(ids, fc, cap)
        assert np.array_equal(got, O.roll_static_keep(ids, fc, cap)), (ids, fc, cap)


def test_roll_static_mask_errors(lib):
    m = (ctypes.c_uint8 * 4)()
    ids = (ctypes.c_int32 * 4)(0, 1, -2, 3)
    assert lib.fkv_roll_static_mask(4, ids, 3, 2, m) == fkv.FKV_ERR_SHAPE
    assert lib.fkv_roll_static_mask(65, ids, 3, 2, m) == fkv.FKV_ERR_SHAPE
    assert lib.fkv_roll_static_mask(4, None, 3, 2, m) == fkv.FKV_ERR_NULL
    assert lib.fkv_roll_static_mask(4, ids, 0, 2, m) == fkv.FKV_ERR_SHAPE
    assert lib.fkv_roll_static_mask(0, None, 3, 2, None) == fkv.FKV_OK


def test_plan_ragged_matches_oracle_offsets(lib):
    """Kept rows for per-head history lengths: the oracle's ragged compression
    on random histories gives the same total."""
    rng = np.random.default_rng(1)
    for trial in range(60):
        H, Fh, Fc, T = int(rng.integers(1, 7)), int(rng.integers(0, 12)), 3, 4
        m = int(rng.integers(0, 6))
        role = rng.integers(0, 2, H).astype(np.uint8)
        fh = rng.integers(0, Fh + 1, H).astype(np.int32)
        mask = np.zeros((H, max(Fh, 1)), dtype=np.uint8)[:, :Fh]
        for h in range(H):
            mask[h, :fh[h]] = rng.integers(0, 2, fh[h])
        d = fkv.make_desc(H, 128, T, Fh, Fc, 2)
        kept, ws = fkv.fkv_plan_ragged(d, fh, role, mask, m)
        want = sum((min(m, fh[h]) if role[h] else int(mask[h].sum())) + Fc for h in range(H)) * T
        assert kept == want, trial
        # the oracle's ragged compaction writes the same number of rows
        off = np.concatenate([[0], np.cumsum(fh.astype(np.int64) * T)])
        D = 8
        hk = np.zeros((int(off[-1]), D), dtype=np.float32)
        cur = np.zeros((Fc * T, H, D), dtype=np.float32)
        q = np.zeros((Fc * T, H, D), dtype=np.float32)
        r = O.compress_ragged(q, hk, hk, off, cur, cur, role, mask, m, T, Fc, 2)
        assert int(r["tok_off"][-1]) == kept


def test_plan_ragged_errors(lib):
    d = fkv.make_desc(2, 128, 8, 6, 3, 2)
    role = np.array([0, 1], dtype=np.uint8)
    mask = np.zeros((2, 6), dtype=np.uint8)
    with pytest.raises(fkv.FkvError, match="hist_frames"):
        fkv.fkv_plan_ragged(d, [7, 2], role, mask, 2)      # beyond desc.hist_frames
    with pytest.raises(fkv.FkvError, match="hist_frames"):
        fkv.fkv_plan_ragged(d, [-1, 2], role, mask, 2)
    mask[0, 4] = 1
    with pytest.raises(fkv.FkvError, match="beyond the head"):
        fkv.fkv_plan_ragged(d, [3, 2], role, mask, 2)      # static mark past its history
    assert fkv.fkv_plan_ragged(d, [5, 0], role, mask, 2)[0] == (1 + 3 + 0 + 3) * 8
    kept = ctypes.c_int64(0)
    assert lib.fkv_plan_ragged(ctypes.byref(d), None, role.ctypes.data, mask.ctypes.data, 2,
                               ctypes.byref(kept), None) == fkv.FKV_ERR_NULL


def test_compress_ragged_and_refresh_argument_errors(lib):
    d = fkv.make_desc(2, 128, 8, 6, 3, 2)
    role = np.array([0, 1], dtype=np.uint8)
    mask = np.zeros((2, 6), dtype=np.uint8)
    fh = np.array([4, 4], dtype=np.int32)
    hist = fkv.FkvCkv(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, None, 1000)
    out = fkv.FkvCkv(0x1000, 0x6000, 0x7000, 0x8000, 0x9000, None, 1000)
    # out sharing a buffer with the history
    st = lib.fkv_compress_ragged(ctypes.byref(d), 0x100, ctypes.byref(hist), fh.ctypes.data,
                                 0x200, 0x300, role.ctypes.data, mask.ctypes.data, 2,
                                 ctypes.byref(out), 0x400, 1 << 20, None)
    assert st == fkv.FKV_ERR_SHAPE
    st = lib.fkv_compress_ragged(ctypes.byref(d), 0x100, ctypes.byref(hist), None, 0x200, 0x300,
                                 role.ctypes.data, mask.ctypes.data, 2, ctypes.byref(out),
                                 0x400, 1 << 20, None)
    assert st == fkv.FKV_ERR_NULL
    st = lib.fkv_compress_ragged(ctypes.byref(d), 0x100, ctypes.byref(hist), fh.ctypes.data,
                                 None, 0x300, role.ctypes.data, mask.ctypes.data, 2,
                                 ctypes.byref(out), 0x400, 1 << 20, None)
    assert st == fkv.FKV_ERR_NULL
    ck = fkv.FkvCkv(None, None, None, None, None, None, 0)
    assert lib.fkv_refresh_current(ctypes.byref(d), 0x100, 0x200, ctypes.byref(ck),
                                   None) == fkv.FKV_ERR_NULL
    assert lib.fkv_refresh_current(ctypes.byref(d), None, 0x200, ctypes.byref(hist),
                                   None) == fkv.FKV_ERR_NULL


# ---- token-granular variant: host plan --------------------------------------

def test_plan_tokens_matches_oracle(lib):
    """Kept rows of the token-granular plan against the oracle's compaction on
    random configurations (zones overlapping, budgets beyond the candidates,
    partial trailing chunks, end tokens covering whole chunks)."""
    rng = np.random.default_rng(7)
    for trial in range(80):
        H, T, Fh, Fc = int(rng.integers(1, 6)), int(rng.integers(1, 9)), \
            int(rng.integers(0, 11)), int(rng.integers(1, 5))
        cfg = fkv.FkvTokenCfg(int(rng.integers(0, 4)), int(rng.integers(0, 5)),
                              int(rng.integers(0, 60)), int(rng.integers(0, 2 * T * Fc + 2)))
        role = rng.integers(0, 2, H).astype(np.uint8)
        d = fkv.make_desc(H, 128, T, Fh, Fc, 2)
        kept, ws = fkv.fkv_plan_tokens(d, cfg, role)
        D = 4
        n_win = (Fh + Fc) * T
        z = np.zeros((n_win, H, D), dtype=np.float32)
        r = O.compress_tokens(z[:Fc * T], z, z, role, T, Fh, Fc, 2, cfg.sink_frames,
                              cfg.recent_frames, cfg.budget_tokens, cfg.boundary_tokens)
        assert kept == int(r["tok_off"][-1]), (trial, H, T, Fh, Fc, list(role))


def test_plan_tokens_errors(lib):
    d = fkv.make_desc(2, 128, 8, 6, 3, 2)
    role = np.array([0, 1], dtype=np.uint8)
    with pytest.raises(fkv.FkvError):
        fkv.fkv_plan_tokens(d, fkv.FkvTokenCfg(-1, 0, 4, 2), role)
    with pytest.raises(fkv.FkvError) as e:
        fkv.fkv_plan_tokens(d, fkv.FkvTokenCfg(1, 1, -4, 2), role)
    assert e.value.status == fkv.FKV_ERR_BUDGET
    kept = ctypes.c_int64(0)
    assert lib.fkv_plan_tokens(ctypes.byref(d), None, role.ctypes.data, ctypes.byref(kept),
                               None) == fkv.FKV_ERR_NULL
    cfg = fkv.FkvTokenCfg(1, 1, 4, 2)
    out = fkv.FkvCkv(0x1000, 0x2000, 0x3000, None, None, None, 1)   # too small
    assert lib.fkv_compress_tokens(ctypes.byref(d), ctypes.byref(cfg), 0x10, 0x20, 0x30,
                                   role.ctypes.data, ctypes.byref(out), None, 0x40, 1 << 20,
                                   None) == fkv.FKV_ERR_CAPACITY


def test_mfma_peak_argument_errors(lib):
    out = ctypes.c_double(0.0)
    assert lib.fkv_mfma_peak(100, None, ctypes.byref(out)) == fkv.FKV_ERR_NULL
    assert lib.fkv_mfma_peak(100, 0x1000, None) == fkv.FKV_ERR_NULL
    assert lib.fkv_mfma_peak(0, 0x1000, ctypes.byref(out)) == fkv.FKV_ERR_SHAPE
