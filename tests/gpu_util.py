"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the CPU oracle to the stated bar."""
import sys

import numpy as np

from hybrid_kv_cache_amd import fkv
from oracle import forcing_kv as O

# Output tolerances: bf16 inputs with fp32 accumulation / fp32 inputs.
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-4
# Beside the absolute bars, the error of every output row (one query of one
# head, D values) relative to that row's norm.  bf16: the output rounding
# alone is up to 2^-9 relative per element and the softmax weights are
# rounded to bf16 for the value product (2^-9 each, averaging out), so rows
# come out near 2e-3; one 64-key tile dropped or counted twice moves the rows
# of its query tile by several percent, far above 1e-2.  fp32: all arithmetic
# in fp32, rows near 1e-6.
BF16_ROW_REL, F32_ROW_REL = 1e-2, 1e-4
# Frame scores (mean softmax mass): the GPU sums exact bf16 products in fp32
# and works in base 2 with fp32 log-sum-exps; each mass comes out within a few
# 1e-7 relative of the float64 value, so the tie band of the selection
# (1e-5 relative) is also the bar for the scores.
SCORE_RTOL = 1e-5


def announce(msg: str) -> None:
    """Name the case on the real stderr before a GPU step (survives capture)."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def require_gpu():
    import pytest
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fkv.load()  # fails loudly when the library is missing


def upload(inp):
    return fkv.to_device(inp.q), fkv.to_device(inp.k), fkv.to_device(inp.v)


def run_compress(w, inp, budget_m=None, mask=None, role=None, q=None, k=None, v=None):
    """Compress one layer on the GPU; returns (desc, ckv, host results)."""
    import torch
    budget_m = w.budget_m if budget_m is None else budget_m
    mask = inp.static_keep_mask if mask is None else mask
    role = inp.head_role if role is None else role
    if q is None:
        q, k, v = upload(inp)
    desc = fkv.desc_for(w)
    ckv = fkv.CompressedKV(desc, role, mask, budget_m)
    announce(f"fkv_compress {w.name} layer={inp.layer} H={w.num_heads} T={w.tokens_per_frame} "
             f"Fh={w.hist_frames} m={budget_m}")
    fkv.fkv_compress(desc, q, k, v, role, mask, budget_m, ckv)
    torch.cuda.synchronize()
    H, Fh = w.num_heads, w.hist_frames
    res = dict(
        seg_off=fkv.to_host(ckv.seg_off),
        tok_off=fkv.to_host(ckv.tok_off),
        seg_idx=fkv.to_host(ckv.seg_idx)[: max(H * Fh, 0)],
        seg_score=fkv.to_host(ckv.seg_score)[: H * Fh].reshape(H, Fh),
    )
    return desc, ckv, (q, k, v), res


def run_attend(desc, q, ckv, n_q, H, D, dtype, workspace="ckv"):
    import torch
    out = torch.empty((n_q, H, D), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device="cuda")
    mode = "per-pair" if workspace is None else "balanced"
    announce(f"fkv_attend Nq={n_q} H={H} D={D} kept={ckv.kept_tokens} {mode}")
    fkv.fkv_attend(desc, q, ckv, out, workspace)
    torch.cuda.synchronize()
    return out


def run_attend_dense(desc, q, k, v, n_q, H, D, dtype, workspace=None):
    import torch
    out = torch.empty((n_q, H, D), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device="cuda")
    mode = "per-pair" if workspace is None else "balanced"
    announce(f"fkv_attend_dense Nq={n_q} H={H} D={D} {mode}")
    fkv.fkv_attend_dense(desc, q, k, v, out, workspace)
    torch.cuda.synchronize()
    return out


def host_f64(t) -> np.ndarray:
    return O.as_f64(fkv.to_host(t))


def check_selection(w, res, oracle_scores, role, mask, budget_m):
    """Kept frames per head: exact outside the cutoff tie band; offsets exact.
    Returns the list of GPU kept frames per head."""
    H, Fh, T, Fc = w.num_heads, w.hist_frames, w.tokens_per_frame, w.cur_frames
    seg_off, seg_idx = res["seg_off"], res["seg_idx"]
    gpu_kept = [np.array(seg_idx[seg_off[h]:seg_off[h + 1]], dtype=np.int64) for h in range(H)]
    for h in range(H):
        g = list(gpu_kept[h])
        assert g == sorted(set(g)), f"head {h}: seg_idx not strictly ascending: {g}"
        if role[h] == O.DYNAMIC:
            assert O.kept_set_valid(g, oracle_scores[h], budget_m), \
                f"head {h}: kept {g} vs oracle scores {oracle_scores[h]}"
        else:
            assert g == list(np.flatnonzero(mask[h])), f"static head {h}: {g}"
    # offsets follow from the kept counts exactly
    _, seg_off_o, tok_off_o = O.offsets(gpu_kept, T, Fc)
    np.testing.assert_array_equal(seg_off, seg_off_o)
    np.testing.assert_array_equal(res["tok_off"], tok_off_o)
    return gpu_kept


def check_scores(res, oracle_scores, role, rtol=SCORE_RTOL):
    """Dynamic heads' scores within rtol of the oracle's (atol only absorbs
    masses below fp32's normal range); NaN for static heads.  Returns the
    largest relative error seen."""
    s = res["seg_score"]
    worst = 0.0
    for h in range(len(role)):
        if role[h] == O.DYNAMIC:
            ref = oracle_scores[h]
            np.testing.assert_allclose(s[h], ref, rtol=rtol, atol=1e-30)
            if ref.size:
                rel = np.abs(s[h] - ref) / np.maximum(np.abs(ref), 1e-30)
                worst = max(worst, float(rel.max()))
        else:
            assert np.isnan(s[h]).all()
    announce(f"scores: max relative error {worst:.3e} (bar {rtol:.0e})")
    return worst


def row_rel_error(got, ref):
    """Per output row (the last axis): ||got - ref|| / ||ref||."""
    num = np.sqrt(np.sum((got - ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(ref ** 2, axis=-1))
    return num / np.maximum(den, 1e-300)


def check_output(got, ref, dtype):
    err = np.abs(got - ref)
    rel = row_rel_error(got, ref)
    if dtype == "bf16":
        assert err.max() <= BF16_MAX_ABS, f"max abs err {err.max()}"
        assert err.mean() <= BF16_MEAN_ABS, f"mean abs err {err.mean()}"
        assert rel.max() <= BF16_ROW_REL, f"row-relative err {rel.max()}"
    else:
        assert err.max() <= F32_MAX_ABS, f"max abs err {err.max()}"
        assert rel.max() <= F32_ROW_REL, f"row-relative err {rel.max()}"
    announce(f"output: max abs {err.max():.3e}, mean abs {err.mean():.3e}, "
             f"max row-relative {rel.max():.3e}")
    return float(err.max()), float(err.mean())
