"""ctypes binding of libfkv.so (C ABI in include/fkv.h).

Argument marshalling only: torch tensors become device pointers and the
current torch stream becomes the hipStream_t; every step of the path runs in
the library's HIP kernels.  Loading fails loudly when the library has not
been built (``python -m hybrid_kv_cache_amd.build``); there is no fallback.

Names mirror the C ABI (EXPORTED below).  ``CompressedKV`` allocates one
layer's ragged cache and workspaces with torch; ``RollingCache`` carries a
layer's compressed cache across chunk steps.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

# FKV_LIB names another build of the same library (the host-sanitizer build
# that the ABI tests also run against); by default the in-tree libfkv.so.
LIB_PATH = os.environ.get("FKV_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                     "libfkv.so")

FKV_OK, FKV_ERR_NULL, FKV_ERR_SHAPE, FKV_ERR_DTYPE, FKV_ERR_BUDGET, \
    FKV_ERR_CAPACITY, FKV_ERR_WORKSPACE, FKV_ERR_HIP = range(8)
FKV_BF16, FKV_F32 = 0, 1
FKV_STATIC, FKV_DYNAMIC = 0, 1

EXPORTED = ("fkv_plan", "fkv_compress", "fkv_compress_attend", "fkv_compress_noalloc",
            "fkv_compress_timed",
            "fkv_plan_ragged", "fkv_compress_ragged", "fkv_refresh_current",
            "fkv_roll_static_mask",
            "fkv_plan_tokens", "fkv_compress_tokens",
            "fkv_compress_fp8", "fkv_attend_fp8",
            "fkv_profile_workspace", "fkv_profile_heads", "fkv_classify_heads",
            "fkv_attend_workspace", "fkv_attend", "fkv_attend_dense",
            "fkv_mfma_peak", "fkv_status_str", "fkv_last_error")


class FkvDesc(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("hist_frames", ctypes.c_int32),
                ("cur_frames", ctypes.c_int32), ("query_stride", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


class FkvCkv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("tok_off", ctypes.c_void_p), ("seg_idx", ctypes.c_void_p),
                ("seg_off", ctypes.c_void_p), ("seg_score", ctypes.c_void_p),
                ("cap_tokens", ctypes.c_int64)]


class FkvTokenCfg(ctypes.Structure):
    _fields_ = [("sink_frames", ctypes.c_int32), ("recent_frames", ctypes.c_int32),
                ("budget_tokens", ctypes.c_int32), ("boundary_tokens", ctypes.c_int32)]


class FkvError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"fkv status {status}: {detail}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfkv.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m hybrid_kv_cache_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.fkv_plan.argtypes = [ctypes.POINTER(FkvDesc), P, P, I32, ctypes.POINTER(I64),
                             ctypes.POINTER(SZ)]
    lib.fkv_compress.argtypes = [ctypes.POINTER(FkvDesc), P, P, P, P, P, I32,
                                 ctypes.POINTER(FkvCkv), P, SZ, P]
    lib.fkv_compress_attend.argtypes = [ctypes.POINTER(FkvDesc), P, P, P, P, P, I32,
                                        ctypes.POINTER(FkvCkv), P, SZ, P, P, SZ, P]
    lib.fkv_compress_noalloc.argtypes = [ctypes.POINTER(FkvDesc), P, P, P, P, P, I32,
                                         ctypes.POINTER(FkvCkv), P]
    lib.fkv_compress_timed.argtypes = [ctypes.POINTER(FkvDesc), P, P, P, P, P, I32,
                                       ctypes.POINTER(FkvCkv), P, SZ, P, P]
    lib.fkv_plan_ragged.argtypes = [ctypes.POINTER(FkvDesc), P, P, P, I32, ctypes.POINTER(I64),
                                    ctypes.POINTER(SZ)]
    lib.fkv_compress_ragged.argtypes = [ctypes.POINTER(FkvDesc), P, ctypes.POINTER(FkvCkv), P,
                                        P, P, P, P, I32, ctypes.POINTER(FkvCkv), P, SZ, P]
    lib.fkv_refresh_current.argtypes = [ctypes.POINTER(FkvDesc), P, P, ctypes.POINTER(FkvCkv), P]
    lib.fkv_roll_static_mask.argtypes = [I32, P, I32, I32, P]
    lib.fkv_plan_tokens.argtypes = [ctypes.POINTER(FkvDesc), ctypes.POINTER(FkvTokenCfg), P,
                                    ctypes.POINTER(I64), ctypes.POINTER(SZ)]
    lib.fkv_compress_tokens.argtypes = [ctypes.POINTER(FkvDesc), ctypes.POINTER(FkvTokenCfg), P,
                                        P, P, P, ctypes.POINTER(FkvCkv), P, P, SZ, P]
    lib.fkv_compress_fp8.argtypes = [ctypes.POINTER(FkvDesc), P, P, P, P, P, I32, P,
                                     ctypes.POINTER(FkvCkv), P, SZ, P]
    lib.fkv_attend_fp8.argtypes = [ctypes.POINTER(FkvDesc), P, ctypes.POINTER(FkvCkv), P, P, P, SZ,
                                   P]
    lib.fkv_profile_workspace.argtypes = [ctypes.POINTER(FkvDesc), ctypes.POINTER(SZ)]
    lib.fkv_profile_heads.argtypes = [ctypes.POINTER(FkvDesc), P, P, P, P, SZ, P]
    lib.fkv_classify_heads.argtypes = [ctypes.POINTER(FkvDesc), P, I32, ctypes.c_float, P, P, P]
    lib.fkv_attend_workspace.argtypes = [ctypes.POINTER(FkvDesc), ctypes.POINTER(SZ)]
    lib.fkv_attend.argtypes = [ctypes.POINTER(FkvDesc), P, ctypes.POINTER(FkvCkv), P, P, SZ, P]
    lib.fkv_attend_dense.argtypes = [ctypes.POINTER(FkvDesc), P, P, P, P, P, SZ, P]
    for name in ("fkv_plan", "fkv_compress", "fkv_compress_attend", "fkv_compress_noalloc",
                 "fkv_compress_timed", "fkv_plan_ragged",
                 "fkv_compress_ragged",
                 "fkv_refresh_current", "fkv_roll_static_mask", "fkv_plan_tokens",
                 "fkv_compress_tokens", "fkv_compress_fp8", "fkv_attend_fp8",
                 "fkv_profile_workspace",
                 "fkv_profile_heads", "fkv_classify_heads", "fkv_attend_workspace",
                 "fkv_attend", "fkv_attend_dense"):
        getattr(lib, name).restype = ctypes.c_int
    lib.fkv_mfma_peak.argtypes = [I32, P, ctypes.POINTER(ctypes.c_double)]
    lib.fkv_mfma_peak.restype = ctypes.c_int
    lib.fkv_status_str.argtypes = [ctypes.c_int]
    lib.fkv_status_str.restype = ctypes.c_char_p
    lib.fkv_last_error.argtypes = []
    lib.fkv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != FKV_OK:
        lib = load()
        raise FkvError(status, f"{lib.fkv_status_str(status).decode()}: "
                               f"{lib.fkv_last_error().decode()}")


def make_desc(num_heads, head_dim, tokens_per_frame, hist_frames, cur_frames,
              query_stride, dtype="bf16", scale=0.0) -> FkvDesc:
    return FkvDesc(num_heads, head_dim, tokens_per_frame, hist_frames, cur_frames,
                   query_stride, float(scale), FKV_BF16 if dtype == "bf16" else FKV_F32)


def desc_for(w, scale: float = 0.0) -> FkvDesc:
    """Descriptor of a hybrid_kv_cache_amd.workloads.Workload."""
    return make_desc(w.num_heads, w.head_dim, w.tokens_per_frame, w.hist_frames,
                     w.cur_frames, w.query_stride, w.dtype, scale)


def _host_u8(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint8))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def fkv_plan(desc: FkvDesc, head_role, static_keep_mask, budget_m: int):
    """Returns (kept_tokens, workspace_bytes)."""
    lib = load()
    role = _host_u8(head_role)
    mask = _host_u8(static_keep_mask)
    kept = ctypes.c_int64(0)
    ws = ctypes.c_size_t(0)
    _check(lib.fkv_plan(ctypes.byref(desc), role.ctypes.data, mask.ctypes.data if mask.size else None,
                        int(budget_m), ctypes.byref(kept), ctypes.byref(ws)))
    return kept.value, ws.value


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def fkv_plan_ragged(desc: FkvDesc, hist_frames, head_role, static_keep_mask, budget_m: int):
    """Returns (kept_tokens, workspace_bytes) for per-head history lengths."""
    lib = load()
    fh = _host_i32(hist_frames)
    role = _host_u8(head_role)
    mask = _host_u8(static_keep_mask)
    kept = ctypes.c_int64(0)
    ws = ctypes.c_size_t(0)
    _check(lib.fkv_plan_ragged(ctypes.byref(desc), fh.ctypes.data, role.ctypes.data,
                               mask.ctypes.data if mask.size else None, int(budget_m),
                               ctypes.byref(kept), ctypes.byref(ws)))
    return kept.value, ws.value


def fkv_roll_static_mask(frame_ids, cur_frames: int, cap: int) -> np.ndarray:
    """Keep mask (uint8) of a static head's history frames in a rolling cache."""
    lib = load()
    ids = _host_i32(frame_ids)
    mask = np.zeros(len(ids), dtype=np.uint8)
    _check(lib.fkv_roll_static_mask(len(ids), ids.ctypes.data if len(ids) else None,
                                    int(cur_frames), int(cap),
                                    mask.ctypes.data if len(ids) else None))
    return mask


class CompressedKV:
    """Device buffers of one layer's compressed cache, allocated with torch.
    With hist_frames (per-head history lengths), sized for fkv_compress_ragged."""

    def __init__(self, desc: FkvDesc, head_role, static_keep_mask, budget_m: int,
                 device="cuda", with_scores: bool = True, hist_frames=None, token_cfg=None,
                 fp8: bool = False):
        import torch
        if token_cfg is not None:
            self.kept_tokens, self.workspace_bytes = fkv_plan_tokens(desc, token_cfg, head_role)
        elif hist_frames is None:
            self.kept_tokens, self.workspace_bytes = fkv_plan(desc, head_role, static_keep_mask,
                                                              budget_m)
        else:
            self.kept_tokens, self.workspace_bytes = fkv_plan_ragged(
                desc, hist_frames, head_role, static_keep_mask, budget_m)
        H, D, Fh = desc.num_heads, desc.head_dim, desc.hist_frames
        dt = torch.bfloat16 if desc.dtype == FKV_BF16 else torch.float32
        if fp8:
            dt = torch.uint8      # e4m3 codes
        self.k = torch.empty((max(self.kept_tokens, 1), D), dtype=dt, device=device)
        self.v = torch.empty((max(self.kept_tokens, 1), D), dtype=dt, device=device)
        self.tok_off = torch.empty(H + 1, dtype=torch.int64, device=device)
        self.seg_idx = torch.empty(max(H * Fh, 1), dtype=torch.int32, device=device)
        self.seg_off = torch.empty(H + 1, dtype=torch.int32, device=device)
        self.seg_score = (torch.empty(max(H * Fh, 1), dtype=torch.float32, device=device)
                          if with_scores else None)
        self.workspace = torch.empty(max(self.workspace_bytes, 1), dtype=torch.uint8,
                                     device=device)
        # Attention workspace (balanced schedule); None where it is not used.
        self.attend_ws = attend_workspace(desc, device)

    def struct(self) -> FkvCkv:
        return FkvCkv(_ptr(self.k), _ptr(self.v), _ptr(self.tok_off), _ptr(self.seg_idx),
                      _ptr(self.seg_off), _ptr(self.seg_score), self.kept_tokens)


def fkv_compress(desc: FkvDesc, q, k_cache, v_cache, head_role, static_keep_mask,
                 budget_m: int, ckv: CompressedKV, stream=None) -> None:
    lib = load()
    role = _host_u8(head_role)
    mask = _host_u8(static_keep_mask)
    out = ckv.struct()
    _check(lib.fkv_compress(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                            role.ctypes.data, mask.ctypes.data if mask.size else None,
                            int(budget_m), ctypes.byref(out), _ptr(ckv.workspace),
                            ckv.workspace_bytes, _stream(stream)))


def fkv_compress_attend(desc: FkvDesc, q, k_cache, v_cache, head_role, static_keep_mask,
                        budget_m: int, ckv: CompressedKV, out, workspace="ckv",
                        stream=None) -> None:
    """fkv_compress then fkv_attend in one call (workspace: the attention
    workspace as for fkv_attend; "ckv" = the one allocated with ckv)."""
    lib = load()
    role = _host_u8(head_role)
    mask = _host_u8(static_keep_mask)
    cs = ckv.struct()
    ws, ws_bytes = _ws(ckv.attend_ws if isinstance(workspace, str) else workspace)
    _check(lib.fkv_compress_attend(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   role.ctypes.data, mask.ctypes.data if mask.size else None,
                                   int(budget_m), ctypes.byref(cs), _ptr(ckv.workspace),
                                   ckv.workspace_bytes, _ptr(out), ws, ws_bytes,
                                   _stream(stream)))


SCRATCH_BYTES = 4 << 20   # FKV_SCRATCH_BYTES


def fkv_compress_noalloc(desc: FkvDesc, q, k_cache, v_cache, head_role, static_keep_mask,
                         budget_m: int, ckv: CompressedKV, stream=None) -> None:
    """fkv_compress on the library's own scratch memory (no workspace)."""
    lib = load()
    role = _host_u8(head_role)
    mask = _host_u8(static_keep_mask)
    out = ckv.struct()
    _check(lib.fkv_compress_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    role.ctypes.data, mask.ctypes.data if mask.size else None,
                                    int(budget_m), ctypes.byref(out), _stream(stream)))


def fkv_compress_ragged(desc: FkvDesc, q, hist: CompressedKV, hist_frames, cur_k, cur_v,
                        head_role, static_keep_mask, budget_m: int, ckv: CompressedKV,
                        stream=None) -> None:
    lib = load()
    fh = _host_i32(hist_frames)
    role = _host_u8(head_role)
    mask = _host_u8(static_keep_mask)
    h = hist.struct()
    out = ckv.struct()
    _check(lib.fkv_compress_ragged(ctypes.byref(desc), _ptr(q), ctypes.byref(h), fh.ctypes.data,
                                   _ptr(cur_k), _ptr(cur_v), role.ctypes.data,
                                   mask.ctypes.data if mask.size else None, int(budget_m),
                                   ctypes.byref(out), _ptr(ckv.workspace), ckv.workspace_bytes,
                                   _stream(stream)))


def fkv_refresh_current(desc: FkvDesc, cur_k, cur_v, ckv: CompressedKV, stream=None) -> None:
    lib = load()
    s = ckv.struct()
    _check(lib.fkv_refresh_current(ctypes.byref(desc), _ptr(cur_k), _ptr(cur_v), ctypes.byref(s),
                                   _stream(stream)))


def fkv_plan_tokens(desc: FkvDesc, cfg: FkvTokenCfg, head_role):
    """Returns (kept_tokens, workspace_bytes) of the token-granular variant."""
    lib = load()
    role = _host_u8(head_role)
    kept = ctypes.c_int64(0)
    ws = ctypes.c_size_t(0)
    _check(lib.fkv_plan_tokens(ctypes.byref(desc), ctypes.byref(cfg), role.ctypes.data,
                               ctypes.byref(kept), ctypes.byref(ws)))
    return kept.value, ws.value


def fkv_compress_tokens(desc: FkvDesc, cfg: FkvTokenCfg, q, k_cache, v_cache, head_role,
                        ckv: CompressedKV, row_src=None, stream=None) -> None:
    lib = load()
    role = _host_u8(head_role)
    out = ckv.struct()
    _check(lib.fkv_compress_tokens(ctypes.byref(desc), ctypes.byref(cfg), _ptr(q), _ptr(k_cache),
                                   _ptr(v_cache), role.ctypes.data, ctypes.byref(out),
                                   _ptr(row_src), _ptr(ckv.workspace), ckv.workspace_bytes,
                                   _stream(stream)))


def _host_f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def fkv_compress_fp8(desc: FkvDesc, q, k_cache, v_cache, head_role, static_keep_mask,
                     budget_m: int, k_scale, v_scale, ckv: CompressedKV, stream=None) -> None:
    """fkv_compress writing an e4m3 cache (ckv allocated with fp8=True)."""
    lib = load()
    role = _host_u8(head_role)
    mask = _host_u8(static_keep_mask)
    sc = _host_f32(np.concatenate([np.ravel(k_scale), np.ravel(v_scale)]))
    out = ckv.struct()
    _check(lib.fkv_compress_fp8(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                role.ctypes.data, mask.ctypes.data if mask.size else None,
                                int(budget_m), sc.ctypes.data, ctypes.byref(out),
                                _ptr(ckv.workspace), ckv.workspace_bytes, _stream(stream)))


def fkv_attend_fp8(desc: FkvDesc, q, ckv: CompressedKV, q_scale, k_scale, v_scale, out,
                   workspace="ckv", stream=None) -> None:
    """workspace: as for fkv_attend ("ckv", None or a device buffer)."""
    lib = load()
    sc = _host_f32(np.concatenate([np.ravel(q_scale), np.ravel(k_scale), np.ravel(v_scale)]))
    s = ckv.struct()
    ws, ws_bytes = _ws(ckv.attend_ws if isinstance(workspace, str) else workspace)
    _check(lib.fkv_attend_fp8(ctypes.byref(desc), _ptr(q), ctypes.byref(s), sc.ctypes.data,
                              _ptr(out), ws, ws_bytes, _stream(stream)))


def fkv_profile_workspace(desc: FkvDesc) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    _check(lib.fkv_profile_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def fkv_profile_heads(desc: FkvDesc, q, k_cache, mass_accum, workspace, stream=None) -> None:
    """Adds this sample's per-(head, frame) mean masses to mass_accum [H, F_tot]
    (a device fp32 tensor)."""
    lib = load()
    _check(lib.fkv_profile_heads(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(mass_accum),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))


def fkv_classify_heads(desc: FkvDesc, mass_sum: np.ndarray, n_calls: int, threshold: float):
    """Host labels from summed masses: (head_role, static_keep_mask, discontinuity)."""
    lib = load()
    H, Fh = desc.num_heads, desc.hist_frames
    m = np.ascontiguousarray(mass_sum, dtype=np.float32)
    role = np.zeros(H, dtype=np.uint8)
    mask = np.zeros((H, max(Fh, 1)), dtype=np.uint8)
    disc = np.zeros(H, dtype=np.float32)
    _check(lib.fkv_classify_heads(ctypes.byref(desc), m.ctypes.data, int(n_calls),
                                  float(threshold), role.ctypes.data, mask.ctypes.data,
                                  disc.ctypes.data))
    return role, mask[:, :Fh], disc


def fkv_attend_workspace(desc: FkvDesc) -> int:
    """Bytes of the optional attention workspace on the current device."""
    lib = load()
    n = ctypes.c_size_t(0)
    _check(lib.fkv_attend_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def attend_workspace(desc: FkvDesc, device="cuda"):
    """A device buffer of fkv_attend_workspace(desc) bytes, or None if 0."""
    import torch
    n = fkv_attend_workspace(desc)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def fkv_compress_timed(desc: FkvDesc, q, k_cache, v_cache, head_role, static_keep_mask,
                       budget_m: int, ckv: CompressedKV, stream=None):
    """fkv_compress with its stage times: (score_ms, select_ms, compact_ms).
    Waits for the device."""
    lib = load()
    role = _host_u8(head_role)
    mask = _host_u8(static_keep_mask)
    out = ckv.struct()
    ms = (ctypes.c_float * 3)()
    _check(lib.fkv_compress_timed(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  role.ctypes.data, mask.ctypes.data if mask.size else None,
                                  int(budget_m), ctypes.byref(out), _ptr(ckv.workspace),
                                  ckv.workspace_bytes, _stream(stream), ms))
    return float(ms[0]), float(ms[1]), float(ms[2])


def fkv_attend(desc: FkvDesc, q, ckv: CompressedKV, out, workspace="ckv",
               stream=None) -> None:
    """workspace: "ckv" (the one CompressedKV allocated), None (one workgroup
    per head and query tile) or a device buffer."""
    lib = load()
    s = ckv.struct()
    ws, ws_bytes = _ws(ckv.attend_ws if isinstance(workspace, str) else workspace)
    _check(lib.fkv_attend(ctypes.byref(desc), _ptr(q), ctypes.byref(s), _ptr(out), ws, ws_bytes,
                          _stream(stream)))


def fkv_attend_dense(desc: FkvDesc, q, k_cache, v_cache, out, workspace=None,
                     stream=None) -> None:
    lib = load()
    ws, ws_bytes = _ws(workspace)
    _check(lib.fkv_attend_dense(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                _ptr(out), ws, ws_bytes, _stream(stream)))


def fkv_mfma_peak(iters: int = 4000) -> float:
    """Measured sustained bf16 MFMA rate of the current device, TFLOP/s."""
    import torch
    lib = load()
    sink = torch.empty(1, dtype=torch.float32, device="cuda")
    out = ctypes.c_double(0.0)
    _check(lib.fkv_mfma_peak(int(iters), _ptr(sink), ctypes.byref(out)))
    return float(out.value)


def fkv_status_str(status: int) -> str:
    return load().fkv_status_str(status).decode()


def fkv_last_error() -> str:
    return load().fkv_last_error().decode()


def to_device(a: np.ndarray, device="cuda"):
    """Host array (float32 values or bf16 bit patterns as uint16) -> torch tensor."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t) -> np.ndarray:
    """torch tensor -> host array (bf16 returned as uint16 bit patterns)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class RollingCache:
    """One layer's compressed cache carried across chunk steps: the cache
    written for chunk c (kept history + chunk c's frames) is chunk c + 1's
    history.  Two device buffers of the largest possible size alternate.

    Host bookkeeping only: each head's history length, and the absolute frame
    ids of static heads' frames (needed for their keep rule, which
    fkv_roll_static_mask applies); dynamic heads' kept ids live on the device
    (seg_idx) and are recorded here as -1.
    """

    def __init__(self, desc: FkvDesc, head_role, budget_m: int, device="cuda",
                 static_cap=None):
        self.desc = desc
        self.role = np.asarray(head_role, dtype=np.uint8)
        self.m = int(budget_m)
        H, Fh, Fc = desc.num_heads, desc.hist_frames, desc.cur_frames
        if self.m > Fh - Fc:
            raise ValueError("a rolling cache needs budget_m <= hist_frames - cur_frames")
        # Static heads keep at most as many frames as their pattern keeps in a
        # plain window of F_h frames (and at most F_h - F_c).
        if static_cap is None:
            static_cap = int(fkv_roll_static_mask(list(range(Fh)), Fc, Fh).sum())
        self.static_cap = min(int(static_cap), Fh - Fc)
        full = np.ones((H, Fh), dtype=np.uint8)
        self.bufs = [CompressedKV(desc, self.role, full, self.m, device=device,
                                  hist_frames=[Fh] * H) for _ in range(2)]
        self.which = 0
        self.chunk = 0
        self.ids = None          # per head: frame ids of the current cache's frames
        self.rows = 0            # rows written by the last step
        self.mask = None

    @property
    def cache(self) -> CompressedKV:
        return self.bufs[self.which]

    def _masks(self, hist_ids):
        H, Fh, Fc = self.desc.num_heads, self.desc.hist_frames, self.desc.cur_frames
        mask = np.zeros((H, Fh), dtype=np.uint8)
        for h in range(H):
            if self.role[h] == 0:
                mk = fkv_roll_static_mask(hist_ids[h], Fc, self.static_cap)
                mask[h, :len(mk)] = mk
        return mask

    def step(self, q, cur_k, cur_v, window_k=None, window_v=None, stream=None):
        """Compress chunk self.chunk.  The first chunk takes the plain window
        (window_k / window_v [N_win, H, D], whose last F_c frames are cur_k /
        cur_v); later chunks take only the current chunk [F_c T, H, D]."""
        d = self.desc
        H, Fh, Fc, T = d.num_heads, d.hist_frames, d.cur_frames, d.tokens_per_frame
        first = Fh + self.chunk * Fc
        if self.chunk == 0:
            hist_ids = [list(range(Fh))] * H
            self.mask = self._masks(hist_ids)
            out = self.bufs[self.which]
            fkv_compress(d, q, window_k, window_v, self.role, self.mask, self.m, out, stream)
            self.rows, _ = fkv_plan(d, self.role, self.mask, self.m)
        else:
            hist_ids = self.ids
            hist_frames = [len(x) for x in hist_ids]
            self.mask = self._masks(hist_ids)
            src = self.bufs[self.which]
            self.which ^= 1
            out = self.bufs[self.which]
            fkv_compress_ragged(d, q, src, hist_frames, cur_k, cur_v, self.role, self.mask,
                                self.m, out, stream)
            self.rows, _ = fkv_plan_ragged(d, hist_frames, self.role, self.mask, self.m)
        new_ids = []
        for h in range(H):
            if self.role[h] == 0:
                kept = [hist_ids[h][f] for f in np.flatnonzero(self.mask[h, :len(hist_ids[h])])]
            else:
                kept = [-1] * min(self.m, len(hist_ids[h]))
            new_ids.append(kept + list(range(first, first + Fc)))
        self.ids = new_ids
        self.chunk += 1
        return self.cache
