"""GPU parity of the FP8 (OCP e4m3) compressed cache: quantizing compaction
(bit-exact codes) and fp8 attention against the CPU oracle, with and without
the attention workspace (one workgroup per pair, or the balanced schedules:
pairs cut into a main part and a tail, or the last round's pairs halved)."""
import numpy as np
import pytest

from hybrid_kv_cache_amd import fkv
from hybrid_kv_cache_amd import workloads as W
from oracle import forcing_kv as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

# Output tolerance of fp8 attention against the oracle's attention on the
# same decoded e4m3 queries, keys and values: the kernel additionally rounds
# every softmax weight to e4m3 (relative error <= 2^-4 each, unbiased), which
# averages out over the keys of a row.
FP8_MAX_ABS, FP8_MEAN_ABS = 3e-2, 3e-3


@pytest.fixture(autouse=True)
def _gpu():
    G.require_gpu()


def head_scales(a, H, D):
    """amax / 448 per head of a token-major [N, H, D] tensor (bf16 bits)."""
    x = np.abs(O.decode_bf16(a)).reshape(-1, H, D).max(axis=(0, 2))
    return np.maximum(x, 1e-6).astype(np.float32) / np.float32(448.0)


def run_fp8(w, inp, rows=None, check_codes=True, workspace="ckv"):
    import torch
    H, D, T, Fh, Fc = w.num_heads, w.head_dim, w.tokens_per_frame, w.hist_frames, w.cur_frames
    ks, vs, qs = head_scales(inp.k, H, D), head_scales(inp.v, H, D), head_scales(inp.q, H, D)
    desc = fkv.desc_for(w)
    q, k, v = fkv.to_device(inp.q), fkv.to_device(inp.k), fkv.to_device(inp.v)
    ckv = fkv.CompressedKV(desc, inp.head_role, inp.static_keep_mask, w.budget_m, fp8=True)
    G.announce(f"fkv_compress_fp8 {w.name} H={H} T={T}")
    fkv.fkv_compress_fp8(desc, q, k, v, inp.head_role, inp.static_keep_mask, w.budget_m, ks, vs,
                         ckv)
    torch.cuda.synchronize()
    ref = O.compress_fp8(inp.q, inp.k, inp.v, inp.head_role, inp.static_keep_mask, w.budget_m,
                         T, Fh, Fc, w.query_stride, ks, vs)
    tok_off = fkv.to_host(ckv.tok_off)
    np.testing.assert_array_equal(tok_off, ref["tok_off"])
    n = int(tok_off[-1])
    k8, v8 = fkv.to_host(ckv.k)[:n], fkv.to_host(ckv.v)[:n]
    if check_codes:
        assert np.array_equal(k8, ref["k8"]), "K codes differ"
        assert np.array_equal(v8, ref["v8"]), "V codes differ"
    out = torch.empty((w.n_q, H, D), dtype=torch.bfloat16, device="cuda")
    G.announce(f"fkv_attend_fp8 {w.name} rows={n} workspace={workspace}")
    fkv.fkv_attend_fp8(desc, q, ckv, qs, ks, vs, out, workspace)
    torch.cuda.synchronize()
    got = G.host_f64(out)
    if rows is not None:
        got = got[rows]
    want = O.attend_fp8(inp.q, k8, v8, tok_off, qs, ks, vs, rows=rows)
    err = np.abs(got - want)
    return err, got, want


@pytest.mark.parametrize("ws", [None, "ckv"])
@pytest.mark.parametrize("T,H,Fh,s,m,nst,seed", [
    (100, 3, 6, 4, 4, 1, 51),      # ragged tiles
    (64, 2, 6, 1, 3, 0, 52),       # exact tiles, all dynamic
    (130, 4, 18, 16, 13, 2, 53),   # 18 history frames
])
def test_fp8_codes_and_attention(T, H, Fh, s, m, nst, seed, ws):
    """With the workspace these few pairs take the split schedule."""
    w = W.small_workload(tokens_per_frame=T, num_heads=H, hist_frames=Fh, query_stride=s,
                         budget_m=m, num_static=nst, seed=seed)
    err, _, _ = run_fp8(w, W.generate_layer(w), workspace=ws)
    assert err.max() <= FP8_MAX_ABS, err.max()
    assert err.mean() <= FP8_MEAN_ABS, err.mean()


def test_fp8_zero_queries_give_exact_value_means():
    """q = 0: every weight is exactly 1 (an e4m3 code), so the output is the
    mean of each head's decoded values to fp32 rounding -- this pins the value
    layout (transposing reads) and the row sums without the weight rounding."""
    w = W.small_workload(tokens_per_frame=90, num_heads=3, hist_frames=6, budget_m=3, seed=54)
    err, got, want = run_fp8(w, W.generate_layer(w, zero_q=True))
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, (err.max(), err.mean())


def test_fp8_late_large_scores_raise_the_reference():
    """Keys of the current chunk aligned with the queries: later tiles' scores
    pass the first tile's by far more than 8 (base 2), so the running
    reference is raised mid-stream and the accumulators rescaled."""
    w = W.small_workload(tokens_per_frame=80, num_heads=3, hist_frames=6, budget_m=3,
                         num_static=1, seed=55)
    inp = W.generate_layer(w)
    qf, kf = inp.as_f32("q"), inp.as_f32("k").copy()
    cur = slice(w.hist_frames * w.tokens_per_frame, None)
    for h in range(w.num_heads):
        u = qf[:, h].mean(axis=0)
        kf[cur, h] = 12.0 * u / max(np.linalg.norm(u), 1e-6) * np.sqrt(w.head_dim) \
            + 0.1 * kf[cur, h]
    inp.k = W.round_to_bf16_bits(kf)
    err, _, _ = run_fp8(w, inp)
    assert err.max() <= FP8_MAX_ABS and err.mean() <= FP8_MEAN_ABS, (err.max(), err.mean())


@pytest.mark.parametrize("T,H,Fh,seed", [
    (2000, 12, 1, 57),    # 564 pairs: 70-71 per XCD, the last 6-7 halved
    (2731, 13, 1, 58),    # 845 pairs: 22-23 halved per XCD
])
def test_fp8_rounds_schedule(T, H, Fh, seed):
    """More (head, query tile) pairs than resident workgroups: with the
    workspace whole pairs run in rounds and the last round's pairs are
    halved, each half with its own reference, merged by the combine kernel
    (which takes the halves' outputs already times the V scale)."""
    w = W.small_workload(tokens_per_frame=T, num_heads=H, hist_frames=Fh, budget_m=Fh,
                         num_static=0, query_stride=7, seed=seed)
    inp = W.generate_layer(w)
    rows = np.random.default_rng(seed).choice(w.n_q, 48, replace=False)
    rows[0], rows[-1] = 0, w.n_q - 1
    for ws in ("ckv", None):
        err, _, _ = run_fp8(w, inp, rows=rows, check_codes=ws == "ckv", workspace=ws)
        assert err.max() <= FP8_MAX_ABS and err.mean() <= FP8_MEAN_ABS, (ws, err.max(), err.mean())


def test_fp8_480p_layer():
    w = W.WORKLOADS["480p_layer"]
    rows = np.random.default_rng(56).choice(w.n_q, 48, replace=False)
    err, _, _ = run_fp8(w, W.generate_layer(w), rows=rows)
    assert err.max() <= FP8_MAX_ABS and err.mean() <= FP8_MEAN_ABS, (err.max(), err.mean())


def test_fp8_random_shapes():
    """Eight seeded random configurations (heads, frame sizes across the
    64-row tiles, history lengths down to none, strides, budgets, mixed
    roles), with and without the attention workspace: codes bit-exact and
    attention within the fp8 bar against the oracle."""
    rng = np.random.default_rng(2026)
    for case in range(8):
        Fh = int(rng.integers(0, 13))
        w = W.small_workload(name=f"fp8_sweep{case}", tokens_per_frame=int(rng.integers(1, 200)),
                             num_heads=int(rng.integers(1, 9)), hist_frames=Fh,
                             cur_frames=int(rng.integers(1, 5)),
                             query_stride=int(rng.integers(1, 9)),
                             budget_m=int(rng.integers(0, Fh + 3)), num_static=0,
                             seed=6000 + case)
        w = W.dataclasses.replace(w, num_static=int(rng.integers(0, w.num_heads + 1)))
        G.announce(f"fp8 sweep case {case}: {w}")
        err, _, _ = run_fp8(w, W.generate_layer(w), workspace="ckv" if case % 2 else None)
        assert err.max() <= FP8_MAX_ABS and err.mean() <= FP8_MEAN_ABS, (case, err.max(),
                                                                         err.mean())


def test_fp8_runs_repeat_bitwise():
    """The fp8 compression and attention (rounds schedule, halved pairs merged
    by the combine kernel) give the same bits on a second run."""
    import torch
    w = W.small_workload(tokens_per_frame=2000, num_heads=12, hist_frames=2, budget_m=1,
                         num_static=4, query_stride=7, seed=59)
    inp = W.generate_layer(w)
    H, D = w.num_heads, w.head_dim
    ks, vs, qs = head_scales(inp.k, H, D), head_scales(inp.v, H, D), head_scales(inp.q, H, D)
    desc = fkv.desc_for(w)
    q, k, v = fkv.to_device(inp.q), fkv.to_device(inp.k), fkv.to_device(inp.v)
    got = []
    for _ in range(2):
        ckv = fkv.CompressedKV(desc, inp.head_role, inp.static_keep_mask, w.budget_m, fp8=True)
        fkv.fkv_compress_fp8(desc, q, k, v, inp.head_role, inp.static_keep_mask, w.budget_m,
                             ks, vs, ckv)
        out = torch.empty((w.n_q, H, D), dtype=torch.bfloat16, device="cuda")
        G.announce(f"fkv_attend_fp8 {w.name} repeat")
        fkv.fkv_attend_fp8(desc, q, ckv, qs, ks, vs, out, "ckv")
        torch.cuda.synchronize()
        got.append((fkv.to_host(ckv.k), fkv.to_host(ckv.v), fkv.to_host(out)))
    for a, b in zip(*got):
        assert np.array_equal(a, b)
