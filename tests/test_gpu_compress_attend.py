"""GPU: fkv_compress_attend (compression and attention of one layer in one
call; with one workgroup per (head, query tile) the heads without scored
frames attend on the library's side stream beside the scoring of the others)
against fkv_compress followed by fkv_attend with the same attention
workspace (none, or the balanced schedules'), bitwise: the compressed cache,
its offsets and the attention output.  One small case is also checked
against the oracle."""
import numpy as np
import pytest

from hybrid_kv_cache_amd import fkv
from hybrid_kv_cache_amd import workloads as W
from oracle import forcing_kv as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.require_gpu()


def _written(w, ckv):
    n = ckv.kept_tokens
    seg_off = fkv.to_host(ckv.seg_off)
    return dict(k=fkv.to_host(ckv.k)[:n], v=fkv.to_host(ckv.v)[:n],
                tok_off=fkv.to_host(ckv.tok_off), seg_off=seg_off,
                seg_idx=fkv.to_host(ckv.seg_idx)[: int(seg_off[-1])],
                seg_score=fkv.to_host(ckv.seg_score)[: w.num_heads * w.hist_frames]
                .view(np.uint32))


def _both(w, inp, role=None, mask=None, ws=None):
    """ws: None (no attention workspace) or "ckv" (the one CompressedKV
    allocates, which selects a balanced schedule where one applies)."""
    import torch
    role = inp.head_role if role is None else role
    mask = inp.static_keep_mask if mask is None else mask
    desc = fkv.desc_for(w)
    q, k, v = G.upload(inp)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ref = fkv.CompressedKV(desc, role, mask, w.budget_m)
    out_ref = torch.empty((w.n_q, w.num_heads, w.head_dim), dtype=dt, device="cuda")
    G.announce(f"fkv_compress + fkv_attend {w.name} roles={list(role)}")
    fkv.fkv_compress(desc, q, k, v, role, mask, w.budget_m, ref)
    fkv.fkv_attend(desc, q, ref, out_ref, ws)
    got = fkv.CompressedKV(desc, role, mask, w.budget_m)
    out = torch.empty_like(out_ref)
    G.announce(f"fkv_compress_attend {w.name}")
    fkv.fkv_compress_attend(desc, q, k, v, role, mask, w.budget_m, got, out, ws)
    torch.cuda.synchronize()
    a, b = _written(w, ref), _written(w, got)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    oa, ob = fkv.to_host(out_ref), fkv.to_host(out)
    assert np.array_equal(oa.view(np.uint8), ob.view(np.uint8)), "attention output"
    return got, out


@pytest.mark.parametrize("ws", [None, "ckv"])
def test_480p_layer_matches_two_calls(ws):
    w = W.WORKLOADS["480p_layer"]
    _both(w, W.generate_layer(w, 0), ws=ws)


def test_1080p_layer_matches_two_calls_with_rounds_schedule():
    """More (head, query tile) pairs than resident workgroups: with the
    workspace the attention runs the rounds schedule after the compression."""
    w = W.WORKLOADS["1080p_layer"]
    _both(w, W.generate_layer(w, 0), ws="ckv")


@pytest.mark.parametrize("ws", [None, "ckv"])
@pytest.mark.parametrize("case", ["mixed", "all_static", "all_dynamic", "no_history"])
def test_small_role_mixes_match_two_calls(case, ws):
    Fh = 0 if case == "no_history" else 7
    w = W.small_workload(tokens_per_frame=150, num_heads=6, hist_frames=Fh, budget_m=min(3, Fh),
                         num_static=2, query_stride=5, seed=71)
    inp = W.generate_layer(w)
    role = inp.head_role.copy()
    if case == "all_static":
        role[:] = fkv.FKV_STATIC
    elif case in ("all_dynamic", "no_history"):
        role[:] = fkv.FKV_DYNAMIC
    _both(w, inp, role=role, ws=ws)


def test_fp32_matches_two_calls_and_oracle():
    w = W.WORKLOADS["tiny_f32"]
    inp = W.generate_layer(w)
    got, out = _both(w, inp)
    scores = O.segment_scores(inp.q, inp.k, inp.head_role, w.tokens_per_frame, w.hist_frames,
                              w.query_stride)
    kept = O.select_frames(scores, inp.head_role, inp.static_keep_mask, w.budget_m)
    k_c, v_c, _, _, tok_off = O.compact(inp.k, inp.v, kept, w.tokens_per_frame, w.hist_frames,
                                        w.cur_frames)
    ref = O.attend(inp.q, k_c, v_c, tok_off)
    G.check_output(G.host_f64(out), ref, w.dtype)


def test_random_shapes_match_two_calls():
    """Twelve seeded random configurations (heads, frame sizes across the
    64-row tiles, history lengths down to none, chunk sizes, strides, budgets
    below and above F_h, mixed roles, bf16 and fp32, with and without the
    attention workspace): one call equals the two calls bitwise."""
    rng = np.random.default_rng(2025)
    for case in range(12):
        dtype = "bf16" if case % 4 else "f32"
        Fh = int(rng.integers(0, 13))
        w = W.small_workload(name=f"ca_sweep{case}_{dtype}", dtype=dtype,
                             head_dim=128 if dtype == "bf16" else 64,
                             tokens_per_frame=int(rng.integers(1, 200)),
                             num_heads=int(rng.integers(1, 9)), hist_frames=Fh,
                             cur_frames=int(rng.integers(1, 5)),
                             query_stride=int(rng.integers(1, 9)),
                             budget_m=int(rng.integers(0, Fh + 3)),
                             num_static=0, seed=5000 + case)
        w = W.dataclasses.replace(w, num_static=int(rng.integers(0, w.num_heads + 1)))
        G.announce(f"one-call sweep case {case}: {w}")
        _both(w, W.generate_layer(w), ws=None if case % 2 else "ckv")
