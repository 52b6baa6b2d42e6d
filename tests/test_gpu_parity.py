"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, at
sizes the oracle finishes in seconds: several tiles per head, ragged tails,
and the degenerate cases of the method."""
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


def full_case(w, inp, budget_m=None, mask=None, role=None, check_dense=True):
    budget_m = w.budget_m if budget_m is None else budget_m
    mask = inp.static_keep_mask if mask is None else mask
    role = inp.head_role if role is None else role
    desc, ckv, (q, k, v), res = G.run_compress(w, inp, budget_m, mask, role)
    scores = O.segment_scores(inp.q, inp.k, role, w.tokens_per_frame, w.hist_frames,
                              w.query_stride)
    G.check_scores(res, scores, role)
    kept = G.check_selection(w, res, scores, role, mask, budget_m)
    k_c, v_c, _, _, tok_off = O.compact(inp.k, inp.v, kept, w.tokens_per_frame,
                                        w.hist_frames, w.cur_frames)
    n = int(tok_off[-1])
    assert np.array_equal(fkv.to_host(ckv.k)[:n], k_c), "compacted K differs"
    assert np.array_equal(fkv.to_host(ckv.v)[:n], v_c), "compacted V differs"
    out = G.run_attend(desc, q, ckv, w.n_q, w.num_heads, w.head_dim, w.dtype)
    ref = O.attend(inp.q, k_c, v_c, tok_off)
    errs = G.check_output(G.host_f64(out), ref, w.dtype)
    if ckv.attend_ws is not None:
        # the other schedule: one workgroup per (head, query tile)
        out1 = G.run_attend(desc, q, ckv, w.n_q, w.num_heads, w.head_dim, w.dtype, None)
        G.check_output(G.host_f64(out1), ref, w.dtype)
    if check_dense:
        dout = G.run_attend_dense(desc, q, k, v, w.n_q, w.num_heads, w.head_dim, w.dtype,
                                  ckv.attend_ws)
        G.check_output(G.host_f64(dout), O.attend_dense(inp.q, inp.k, inp.v), w.dtype)
    return desc, ckv, (q, k, v), out, kept, errs


def test_tiny_f32_workload():
    w = W.WORKLOADS["tiny_f32"]
    full_case(w, W.generate_layer(w))


@pytest.mark.parametrize("T,H,Fh,s,m,nst,seed", [
    (100, 3, 6, 4, 4, 1, 7),      # 300 queries, 900-key window: ragged tiles
    (37, 5, 8, 3, 5, 2, 8),       # tiny frames, many heads
    (64, 2, 6, 1, 3, 0, 9),       # every query scored, all dynamic, exact tiles
    (130, 4, 18, 16, 13, 2, 10),  # 18 history frames as in the video workloads
])
def test_small_bf16(T, H, Fh, s, m, nst, seed):
    w = W.small_workload(tokens_per_frame=T, num_heads=H, hist_frames=Fh, query_stride=s,
                         budget_m=m, num_static=nst, seed=seed)
    full_case(w, W.generate_layer(w))


def test_small_f32_d128():
    w = W.small_workload(name="small_f32", dtype="f32", head_dim=128, tokens_per_frame=40,
                         num_heads=3, hist_frames=5, query_stride=5, budget_m=2, seed=11)
    full_case(w, W.generate_layer(w))


def test_keep_all_equals_dense_bitwise():
    """Keep-all budgets and all-ones masks: the compressed cache is the whole
    window in order, so attend and attend_dense run the same arithmetic."""
    w = W.small_workload(tokens_per_frame=70, num_heads=3, hist_frames=6, budget_m=6, seed=12)
    inp = W.generate_layer(w)
    mask = np.ones_like(inp.static_keep_mask)
    desc, ckv, (q, k, v), out, kept, _ = full_case(w, inp, budget_m=6, mask=mask,
                                                   check_dense=False)
    assert all(list(kh) == list(range(6)) for kh in kept)
    # same schedule on both sides (the balanced one, where there is one)
    dout = G.run_attend_dense(desc, q, k, v, w.n_q, w.num_heads, w.head_dim, w.dtype,
                              ckv.attend_ws)
    assert np.array_equal(fkv.to_host(out), fkv.to_host(dout))
    out1 = G.run_attend(desc, q, ckv, w.n_q, w.num_heads, w.head_dim, w.dtype, None)
    dout1 = G.run_attend_dense(desc, q, k, v, w.n_q, w.num_heads, w.head_dim, w.dtype, None)
    assert np.array_equal(fkv.to_host(out1), fkv.to_host(dout1))


def test_budget_above_history_keeps_all():
    w = W.small_workload(tokens_per_frame=20, num_heads=2, hist_frames=4, budget_m=9,
                         num_static=0, seed=13)
    _, _, _, _, kept, _ = full_case(w, W.generate_layer(w), budget_m=9)
    assert all(list(kh) == [0, 1, 2, 3] for kh in kept)


def test_zero_budget_and_empty_mask_attend_current_chunk_only():
    w = W.small_workload(tokens_per_frame=50, num_heads=3, hist_frames=6, budget_m=0, seed=14)
    inp = W.generate_layer(w)
    mask = np.zeros_like(inp.static_keep_mask)
    desc, ckv, (q, k, v), out, kept, _ = full_case(w, inp, budget_m=0, mask=mask,
                                                   check_dense=False)
    assert all(len(kh) == 0 for kh in kept)
    cur = slice(w.hist_frames * w.tokens_per_frame, None)
    ref = O.attend_dense(inp.q, inp.k[cur], inp.v[cur])
    G.check_output(G.host_f64(out), ref, w.dtype)


def test_zero_queries_tie_break_lowest_frames():
    """q = 0: every frame receives exactly the same mass, and the kept set of
    every dynamic head is frames 0..m-1 on both sides."""
    for dtype, D in (("bf16", 128), ("f32", 64)):
        w = W.small_workload(name=f"zeroq_{dtype}", dtype=dtype, head_dim=D,
                             tokens_per_frame=90, num_heads=3, hist_frames=7, budget_m=4,
                             num_static=1, seed=15)
        inp = W.generate_layer(w, zero_q=True)
        desc, ckv, _, res = G.run_compress(w, inp)
        for h in range(w.num_heads):
            if inp.head_role[h] == O.DYNAMIC:
                s = res["seg_score"][h]
                assert np.all(s == s[0]), s
                kh = res["seg_idx"][res["seg_off"][h]:res["seg_off"][h + 1]]
                assert list(kh) == [0, 1, 2, 3]


def test_no_history_single_head_single_token_frames():
    w = W.small_workload(tokens_per_frame=1, num_heads=1, hist_frames=0, cur_frames=3,
                         budget_m=2, num_static=0, query_stride=1, seed=16)
    full_case(w, W.generate_layer(w))
    w = W.small_workload(tokens_per_frame=1, num_heads=1, hist_frames=5, cur_frames=1,
                         budget_m=2, num_static=0, query_stride=1, seed=17)
    full_case(w, W.generate_layer(w))


def test_max_heads_and_frames():
    w = W.small_workload(tokens_per_frame=3, num_heads=64, hist_frames=64, cur_frames=8,
                         budget_m=40, num_static=20, query_stride=2, seed=18)
    full_case(w, W.generate_layer(w))


def test_deterministic_across_runs():
    w = W.small_workload(tokens_per_frame=100, num_heads=3, hist_frames=6, seed=19)
    inp = W.generate_layer(w)
    outs = []
    for _ in range(2):
        desc, ckv, (q, k, v), res = G.run_compress(w, inp)
        out = G.run_attend(desc, q, ckv, w.n_q, w.num_heads, w.head_dim, w.dtype)
        outs.append((res["seg_score"].copy(), fkv.to_host(ckv.k).copy(), fkv.to_host(out)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b, equal_nan=True) if a.dtype.kind == "f" else np.array_equal(a, b)


def test_late_frames_with_much_larger_scores():
    """Keys of the current chunk scaled up so that their logits exceed the
    first tiles' by far more than 2^64 in weight: the running reference must
    be raised mid-stream (score and attention kernels) with exact results."""
    for dtype, D in (("bf16", 128), ("f32", 64)):
        w = W.small_workload(name=f"late_{dtype}", dtype=dtype, head_dim=D,
                             tokens_per_frame=80, num_heads=3, hist_frames=6, budget_m=3,
                             num_static=1, seed=21)
        inp = W.generate_layer(w)
        q = inp.as_f32("q")
        k = inp.as_f32("k").copy()
        cur = slice(w.hist_frames * w.tokens_per_frame, None)
        # align the current chunk's keys with each head's mean query, x40
        for h in range(w.num_heads):
            u = q[:, h].mean(axis=0)
            k[cur, h] = 40.0 * u / max(np.linalg.norm(u), 1e-6) * np.sqrt(D) + 0.1 * k[cur, h]
        if dtype == "bf16":
            inp.k = W.round_to_bf16_bits(k)
        else:
            inp.k = k.astype(np.float32)
        full_case(w, inp)


@pytest.mark.parametrize("T,H,Fh,Fc,seed", [
    (10, 1, 2, 1, 31),     # one pair of one tile: not cut (the tail takes it whole)
    (100, 1, 3, 1, 36),    # one pair of 7 tiles: cut in halves
    (300, 1, 40, 2, 32),   # 5 pairs x 197 tiles, one tail workgroup per pair
    (257, 7, 9, 3, 33),    # 49 pairs x 49 tiles
    (1560, 12, 18, 3, 34), # 480P window, 444 pairs: per pair even with a workspace
])
def test_split_schedule(T, H, Fh, Fc, seed):
    """With a workspace and at most one (head, query tile) pair per CU,
    attention cuts pairs into a main part and a tail run by different
    workgroups and merges the two partial results: the result matches the
    oracle and the one-workgroup-per-pair schedule."""
    w = W.small_workload(tokens_per_frame=T, num_heads=H, hist_frames=Fh, cur_frames=Fc,
                         budget_m=min(3, Fh), num_static=0, query_stride=7, seed=seed)
    inp = W.generate_layer(w)
    desc = fkv.desc_for(w)
    q, k, v = (fkv.to_device(inp.q), fkv.to_device(inp.k), fkv.to_device(inp.v))
    ws = fkv.attend_workspace(desc)
    assert ws is not None
    if w.n_q * w.n_win * H <= 100_000_000:
        ref = O.attend_dense(inp.q, inp.k, inp.v)
        rows = None
    else:  # sampled rows, each computed by the oracle one by one
        rows = np.random.default_rng(seed).choice(w.n_q, 48, replace=False)
        ref = O.attend_dense(inp.q, inp.k, inp.v, rows=rows)
    outs = []
    for workspace in (ws, None):
        out = G.run_attend_dense(desc, q, k, v, w.n_q, H, w.head_dim, w.dtype, workspace)
        got = G.host_f64(out)
        G.check_output(got if rows is None else got[rows], ref, w.dtype)
        outs.append(got)
    # the two schedules differ only by the order of fp32 sums: at most a
    # couple of bf16 rounding steps apart
    assert np.max(np.abs(outs[0] - outs[1])) <= 2e-2


@pytest.mark.parametrize("T,H,Fh,Fc,seed", [
    (2000, 12, 2, 3, 41),  # 564 pairs: 70-71 per XCD, the last 6-7 halved (2 rem <= 64)
    (2731, 13, 1, 3, 42),  # 845 pairs: 105-106 per XCD, 22-23 halved (2 rem > 64)
    (130, 64, 0, 8, 43),   # 576 pairs of 17 tiles, 8 halved per XCD
])
def test_rounds_schedule(T, H, Fh, Fc, seed):
    """With a workspace and more (head, query tile) pairs than resident
    workgroups, whole pairs run in rounds and the pairs left for the last
    round are halved so that it is full: the result matches the oracle on
    sampled rows and the one-workgroup-per-pair schedule everywhere."""
    w = W.small_workload(tokens_per_frame=T, num_heads=H, hist_frames=Fh, cur_frames=Fc,
                         budget_m=min(3, Fh), num_static=0, query_stride=7, seed=seed)
    inp = W.generate_layer(w)
    desc = fkv.desc_for(w)
    q, k, v = (fkv.to_device(inp.q), fkv.to_device(inp.k), fkv.to_device(inp.v))
    ws = fkv.attend_workspace(desc)
    assert ws is not None
    rows = np.random.default_rng(seed).choice(w.n_q, 48, replace=False)
    rows[0], rows[-1] = 0, w.n_q - 1
    ref = O.attend_dense(inp.q, inp.k, inp.v, rows=rows)
    outs = []
    for workspace in (ws, None):
        out = G.run_attend_dense(desc, q, k, v, w.n_q, H, w.head_dim, w.dtype, workspace)
        got = G.host_f64(out)
        G.check_output(got[rows], ref, w.dtype)
        outs.append(got)
    # whole pairs are computed identically; halved pairs differ from the
    # per-pair result by the order of fp32 sums only
    assert np.max(np.abs(outs[0] - outs[1])) <= 2e-2



def test_rounds_schedule_changes_only_the_halved_pairs():
    """Each attention schedule gives the same bits on every run, and the
    rounds schedule touches only the pairs it halves.  Workgroup b runs on
    XCD b % 8; XCD x takes the contiguous eighth [p_lo, p_lo + n) of the
    (head, 128-query tile) pairs, runs them in rounds of slots = 2 * CUs / 8
    workgroups and halves the last s of them, s = rem if 2 rem <= slots else
    slots - rem (rem = n mod slots), so that the last round is full.  Every
    other pair must equal the one-workgroup-per-pair result bit for bit."""
    import torch
    w = W.small_workload(tokens_per_frame=2000, num_heads=12, hist_frames=2, cur_frames=3,
                         budget_m=2, num_static=0, query_stride=7, seed=44)
    inp = W.generate_layer(w)
    desc = fkv.desc_for(w)
    q, k, v = (fkv.to_device(inp.q), fkv.to_device(inp.k), fkv.to_device(inp.v))
    ws = fkv.attend_workspace(desc)
    outs = []
    for workspace in (ws, None):
        runs = [fkv.to_host(G.run_attend_dense(desc, q, k, v, w.n_q, w.num_heads, w.head_dim,
                                               w.dtype, workspace)) for _ in range(2)]
        assert np.array_equal(runs[0], runs[1]), "two runs of one schedule differ"
        outs.append(runs[0])
    ntq = -(-w.n_q // 128)
    pairs = ntq * w.num_heads
    slots = 2 * torch.cuda.get_device_properties(0).multi_processor_count // 8
    assert pairs > 8 * slots   # more pairs than resident workgroups: rounds
    halved = set()
    for x in range(8):
        p_lo = pairs * x // 8
        n = pairs * (x + 1) // 8 - p_lo
        rem = n % slots
        s = 0 if rem == 0 else (rem if 2 * rem <= slots else slots - rem)
        halved.update(range(p_lo + n - s, p_lo + n))
    assert 0 < len(halved) < pairs
    changed = 0
    for p in range(pairs):
        h, qt = divmod(p, ntq)
        rows = slice(qt * 128, min((qt + 1) * 128, w.n_q))
        if not np.array_equal(outs[0][rows, h], outs[1][rows, h]):
            assert p in halved, f"whole pair {p} (head {h}, tile {qt}) changed"
            changed += 1
    G.announce(f"{changed} of {len(halved)} halved pairs differ in some bit; "
               f"{pairs - len(halved)} whole pairs identical")

def test_attend_workspace_too_small_is_rejected():
    w = W.small_workload(tokens_per_frame=20, num_heads=2, hist_frames=3, seed=35)
    inp = W.generate_layer(w)
    desc = fkv.desc_for(w)
    q, k, v = (fkv.to_device(inp.q), fkv.to_device(inp.k), fkv.to_device(inp.v))
    import torch
    n = fkv.fkv_attend_workspace(desc)
    small = torch.empty(n - 256, dtype=torch.uint8, device="cuda")
    out = torch.empty((w.n_q, w.num_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        fkv.fkv_attend_dense(desc, q, k, v, out, small)


def test_random_shapes_sweep():
    """Twenty seeded random configurations (heads, frame sizes across the
    64-row tiles, history lengths down to none, chunk sizes, strides, budgets
    below and above F_h, mixed roles, bf16 and fp32): selection, offsets,
    compacted rows, compressed and full-KV attention against the oracle."""
    rng = np.random.default_rng(2024)
    for case in range(20):
        dtype = "bf16" if case % 3 else "f32"
        Fh = int(rng.integers(0, 13))
        w = W.small_workload(name=f"sweep{case}_{dtype}", dtype=dtype,
                             head_dim=128 if dtype == "bf16" else 64,
                             tokens_per_frame=int(rng.integers(1, 150)),
                             num_heads=int(rng.integers(1, 9)), hist_frames=Fh,
                             cur_frames=int(rng.integers(1, 5)),
                             query_stride=int(rng.integers(1, 9)),
                             budget_m=int(rng.integers(0, Fh + 3)),
                             num_static=0, seed=3000 + case)
        w = W.dataclasses.replace(w, num_static=int(rng.integers(0, w.num_heads + 1)))
        G.announce(f"sweep case {case}: {w}")
        full_case(w, W.generate_layer(w))



def test_random_wide_windows_sweep():
    """Ten seeded random configurations with long windows (up to 40 history
    and 8 current frames, so windows past 24 frames take the selection's
    4-wave path), frames up to 300 tokens and up to 12 heads, bf16 and fp32
    with D 64 or 128: the same checks as the sweep above."""
    rng = np.random.default_rng(77001)
    for case in range(10):
        dtype = "f32" if case % 4 == 3 else "bf16"
        D = 128 if dtype == "bf16" else int(rng.choice([64, 128]))
        Fh, H = int(rng.integers(0, 41)), int(rng.integers(1, 13))
        w = W.small_workload(name=f"wide{case}_{dtype}", dtype=dtype, head_dim=D,
                             tokens_per_frame=int(rng.integers(1, 301)), num_heads=H,
                             hist_frames=Fh, cur_frames=int(rng.integers(1, 9)),
                             query_stride=int(rng.integers(1, 13)),
                             budget_m=int(rng.integers(0, Fh + 3)), num_static=0,
                             seed=8000 + case)
        w = W.dataclasses.replace(w, num_static=int(rng.integers(0, H + 1)))
        G.announce(f"wide sweep case {case}: {w}")
        full_case(w, W.generate_layer(w))

def test_compress_timed_matches_compress():
    """The measurement helper runs the same kernels: identical cache, offsets
    and selection, and positive stage times (scoring 0 without dynamic heads)."""
    import torch
    w = W.small_workload(tokens_per_frame=90, num_heads=4, hist_frames=6, seed=61)
    inp = W.generate_layer(w)
    desc, ckv, (q, k, v), _ = G.run_compress(w, inp)
    ckv2 = fkv.CompressedKV(desc, inp.head_role, inp.static_keep_mask, w.budget_m)
    ms = fkv.fkv_compress_timed(desc, q, k, v, inp.head_role, inp.static_keep_mask,
                                w.budget_m, ckv2)
    torch.cuda.synchronize()
    n = ckv.kept_tokens
    n_seg = int(fkv.to_host(ckv.seg_off)[-1])
    for a, b, cnt in ((ckv.k, ckv2.k, n), (ckv.v, ckv2.v, n),
                      (ckv.tok_off, ckv2.tok_off, None), (ckv.seg_off, ckv2.seg_off, None),
                      (ckv.seg_idx, ckv2.seg_idx, n_seg)):
        assert np.array_equal(fkv.to_host(a)[:cnt], fkv.to_host(b)[:cnt])
    assert all(t > 0 for t in ms), ms
    role0 = np.zeros(w.num_heads, dtype=np.uint8)
    ckv3 = fkv.CompressedKV(desc, role0, inp.static_keep_mask, w.budget_m)
    ms0 = fkv.fkv_compress_timed(desc, q, k, v, role0, inp.static_keep_mask, w.budget_m, ckv3)
    assert ms0[1] > 0 and ms0[2] > 0 and ms0[0] == 0.0


def test_mfma_peak_calibration_is_plausible():
    """The calibration kernel reports a bf16 MFMA rate between half and the
    whole of the datasheet's 2.5 PFLOP/s."""
    tf = fkv.fkv_mfma_peak(iters=2000)
    assert 1250.0 < tf <= 2600.0, tf


def test_no_writes_past_the_outputs():
    """Every output buffer gets 4 KiB of sentinel bytes past its end: the
    compressed K/V (bf16 and e4m3), offsets, selection, scores, attention
    output and the token variant's row sources are written only within their
    documented extent."""
    import torch
    w = W.small_workload(tokens_per_frame=100, num_heads=5, hist_frames=9, budget_m=4,
                         num_static=2, query_stride=3, seed=71)
    inp = W.generate_layer(w)
    desc = fkv.desc_for(w)
    q, k, v = fkv.to_device(inp.q), fkv.to_device(inp.k), fkv.to_device(inp.v)
    pad = 4096

    def padded(t, n_elems):
        """A flat tensor of n_elems + pad bytes' worth, sentinel-filled, and its head view."""
        per = t.element_size()
        raw = torch.full((n_elems * per + pad,), 0xA5, dtype=torch.uint8, device="cuda")
        return raw, raw[:n_elems * per].view(t.dtype)

    ckv = fkv.CompressedKV(desc, inp.head_role, inp.static_keep_mask, w.budget_m)
    raws = []
    for name in ("k", "v", "tok_off", "seg_idx", "seg_off", "seg_score"):
        t = getattr(ckv, name)
        raw, view = padded(t, t.numel())
        setattr(ckv, name, view.view(t.shape))
        raws.append((name, raw, t.numel() * t.element_size()))
    fkv.fkv_compress(desc, q, k, v, inp.head_role, inp.static_keep_mask, w.budget_m, ckv)
    out_raw, out = padded(torch.empty(0, dtype=torch.bfloat16), w.n_q * w.num_heads * w.head_dim)
    fkv.fkv_attend(desc, q, ckv, out.view(w.n_q, w.num_heads, w.head_dim))
    # e4m3 cache
    c8 = fkv.CompressedKV(desc, inp.head_role, inp.static_keep_mask, w.budget_m, fp8=True)
    for name in ("k", "v"):
        t = getattr(c8, name)
        raw, view = padded(t, t.numel())
        setattr(c8, name, view.view(t.shape))
        raws.append(("fp8 " + name, raw, t.numel()))
    sc = np.full(w.num_heads, 0.02, dtype=np.float32)
    fkv.fkv_compress_fp8(desc, q, k, v, inp.head_role, inp.static_keep_mask, w.budget_m, sc,
                         sc, c8)
    # token variant row sources
    cfg = fkv.FkvTokenCfg(1, 2, 150, 20)
    ct = fkv.CompressedKV(desc, inp.head_role, None, 0, token_cfg=cfg)
    src_raw, src = padded(torch.empty(0, dtype=torch.int32), ct.kept_tokens)
    fkv.fkv_compress_tokens(desc, cfg, q, k, v, inp.head_role, ct, src)
    torch.cuda.synchronize()
    for name, raw, nbytes in raws + [("out", out_raw, out.numel() * 2),
                                      ("row_src", src_raw, ct.kept_tokens * 4)]:
        tail = fkv.to_host(raw)[nbytes:]
        assert (tail == 0xA5).all(), f"{name}: bytes written past the end"
