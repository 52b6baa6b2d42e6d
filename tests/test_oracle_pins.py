"""Pins of the CPU oracle against facts other than itself (no GPU).

Each test below fixes the oracle to something the method or the mathematics
decides independently of the oracle's own code: conservation laws, closed
forms, brute-force enumeration, or a library routine (torch's
scaled_dot_product_attention in float64) computing the same quantity by a
different route.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import forcing_kv as O
from hybrid_kv_cache_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, H=3, D=16, T=5, Fh=4, Fc=2, dyn=None):
    N = (Fh + Fc) * T
    q = rng.standard_normal((Fc * T, H, D))
    k = rng.standard_normal((N, H, D))
    v = rng.standard_normal((N, H, D))
    role = np.ones(H, np.uint8) if dyn is None else np.asarray(dyn, np.uint8)
    return q, k, v, role


def _sdpa(qh, kh, vh, scale):
    """torch library attention in float64: [n, D] x [N, D] x [N, E]."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qh)[None, None], torch.from_numpy(kh)[None, None],
        torch.from_numpy(vh)[None, None], scale=scale)
    return out[0, 0].numpy()


# ---------------------------------------------------------------- scoring

def test_masses_sum_to_one_over_whole_window():
    rng = np.random.default_rng(0)
    q, k, _, _ = _rand_case(rng, H=2, D=16, T=7, Fh=5, Fc=3)
    for h in range(2):
        mass = O.frame_masses(q[:, h], k[:, h], 7, 3, 0.25)
        assert mass.shape == (math.ceil(21 / 3), 8)
        np.testing.assert_allclose(mass.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert (mass > 0).all()


def test_masses_equal_library_attention_onto_frame_indicators():
    """mass[i, f] = sum over frame f of softmax weights = attention with values
    equal to the one-hot frame indicator of each key; torch's SDPA computes it
    by another route (catches a wrong scale, a wrong softmax domain or a wrong
    frame boundary)."""
    rng = np.random.default_rng(1)
    T, Fh, Fc, D, s = 6, 4, 3, 32, 5
    q, k, _, _ = _rand_case(rng, H=1, D=D, T=T, Fh=Fh, Fc=Fc)
    q *= 2.0
    frame_of_key = np.arange((Fh + Fc) * T) // T
    indicator = np.eye(Fh + Fc)[frame_of_key]
    rows = np.arange(0, Fc * T, s)
    ref = _sdpa(q[rows, 0], k[:, 0], indicator, 1 / math.sqrt(D))
    got = O.frame_masses(q[:, 0], k[:, 0], T, s, O.logit_scale(D))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_scores_are_mean_of_history_masses_via_library():
    rng = np.random.default_rng(2)
    T, Fh, Fc, D, s = 4, 5, 3, 16, 2
    q, k, _, role = _rand_case(rng, H=3, D=D, T=T, Fh=Fh, Fc=Fc, dyn=[1, 0, 1])
    sc = O.segment_scores(q, k, role, T, Fh, s)
    assert np.isnan(sc[1]).all()
    indicator = np.eye(Fh + Fc)[np.arange((Fh + Fc) * T) // T]
    rows = np.arange(0, Fc * T, s)
    for h in (0, 2):
        ref = _sdpa(q[rows, h], k[:, h], indicator, 1 / math.sqrt(D))[:, :Fh].mean(axis=0)
        np.testing.assert_allclose(sc[h], ref, rtol=0, atol=1e-12)


def test_constant_key_frames_closed_form():
    """Keys of frame f all equal c_f: each frame holds T equal logits, so the
    per-frame mass is the softmax over frames of scale * q . c_f."""
    rng = np.random.default_rng(3)
    T, Fh, Fc, D = 9, 4, 2, 16
    c = rng.standard_normal((Fh + Fc, D)) * 1.5
    k = np.repeat(c, T, axis=0)[:, None, :]
    q = rng.standard_normal((Fc * T, 1, D))
    mass = O.frame_masses(q[:, 0], k[:, 0], T, 1, 1 / math.sqrt(D))
    z = q[:, 0] @ c.T / math.sqrt(D)
    from scipy.special import softmax
    np.testing.assert_allclose(mass, softmax(z, axis=1), rtol=0, atol=1e-12)


def test_zero_queries_give_uniform_masses_and_lowest_index_ties():
    """q = 0: every logit is 0, so every frame gets mass exactly T/N_win =
    1/F_total; all scores tie exactly and the tie-break keeps frames 0..m-1."""
    rng = np.random.default_rng(4)
    T, Fh, Fc, D = 5, 6, 3, 8
    _, k, v, role = _rand_case(rng, H=2, D=D, T=T, Fh=Fh, Fc=Fc)
    q = np.zeros((Fc * T, 2, D))
    sc = O.segment_scores(q, k, role, T, Fh, 2)
    np.testing.assert_allclose(sc, 1.0 / (Fh + Fc), rtol=0, atol=1e-15)
    for m in range(Fh + 2):
        kept = O.select_frames(sc, role, np.zeros((2, Fh), np.uint8), m)
        for h in range(2):
            assert list(kept[h]) == list(range(min(m, Fh)))


def test_dominant_frame_takes_all_mass():
    rng = np.random.default_rng(5)
    T, Fh, Fc, D = 4, 5, 2, 16
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = np.tile(u, (Fc * T, 1))[:, None, :]
    k = 0.01 * rng.standard_normal(((Fh + Fc) * T, 1, D))
    k[2 * T:3 * T, 0] = 40.0 * math.sqrt(D) * u
    sc = O.segment_scores(q, k, np.ones(1, np.uint8), T, Fh, 1)
    assert sc[0, 2] > 1 - 1e-12
    assert sc[0].sum() <= 1 + 1e-12


def test_permuting_tokens_within_a_frame_changes_nothing():
    rng = np.random.default_rng(6)
    T, Fh, Fc, D, s = 6, 4, 2, 16, 3
    q, k, v, role = _rand_case(rng, H=2, D=D, T=T, Fh=Fh, Fc=Fc)
    perm = np.concatenate([f * T + rng.permutation(T) for f in range(Fh + Fc)])
    s1 = O.segment_scores(q, k, role, T, Fh, s)
    s2 = O.segment_scores(q, k[perm], role, T, Fh, s)
    np.testing.assert_allclose(s1, s2, rtol=1e-13, atol=0)
    mask = np.ones((2, Fh), np.uint8)
    a = O.compress(q, k, v, role, mask, 2, T, Fh, Fc, s)
    b = O.compress(q, k[perm], v[perm], role, mask, 2, T, Fh, Fc, s)
    assert [list(x) for x in a["kept"]] == [list(x) for x in b["kept"]]
    oa = O.attend(q, a["k_c"], a["v_c"], a["tok_off"])
    ob = O.attend(q, b["k_c"], b["v_c"], b["tok_off"])
    np.testing.assert_allclose(oa, ob, rtol=0, atol=1e-13)


def test_strided_sample_is_every_sth_flat_query():
    assert list(O.sampled_query_rows(10, 4)) == [0, 4, 8]
    assert len(O.sampled_query_rows(4680, 16)) == 293
    assert len(O.sampled_query_rows(24480, 32)) == 765
    # scoring with stride s equals scoring the s-th rows with stride 1
    rng = np.random.default_rng(7)
    q, k, _, role = _rand_case(rng, H=1, D=8, T=5, Fh=3, Fc=2)
    a = O.segment_scores(q, k, role, 5, 3, 3)
    b = O.segment_scores(q[::3], k, role, 5, 3, 1)
    np.testing.assert_allclose(a, b, rtol=0, atol=0)


# -------------------------------------------------------------- selection

def _brute_force_topm(score_row, m):
    """Enumerate every m-subset; keep the largest score sum, and among equal
    sums the lexicographically smallest index set.  Sums are compared exactly
    (as fractions), so equal-sum subsets are recognised as such."""
    from fractions import Fraction
    f_h = len(score_row)
    m = min(m, f_h)
    best, best_key = None, None
    for sub in itertools.combinations(range(f_h), m):
        key = (-sum(Fraction(float(score_row[i])) for i in sub), sub)
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return list(best)


@pytest.mark.parametrize("seed", range(20))
def test_dynamic_selection_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    f_h = int(rng.integers(1, 9))
    # small integers: exact ties occur often and subset sums are exact
    scores = rng.integers(0, 4, f_h).astype(np.float64)
    for m in range(f_h + 2):
        assert list(O.select_dynamic(scores, m)) == _brute_force_topm(scores, m)


def test_static_selection_is_mask_and_budget_ignored():
    mask = np.array([[1, 0, 1, 1, 0, 1], [0, 0, 0, 0, 0, 0]], np.uint8)
    role = np.array([O.STATIC, O.STATIC], np.uint8)
    for m in (0, 3, 10):
        kept = O.select_frames(np.full((2, 6), np.nan), role, mask, m)
        assert list(kept[0]) == [0, 2, 3, 5] and list(kept[1]) == []


def test_negative_budget_rejected():
    with pytest.raises(ValueError):
        O.select_frames(np.zeros((1, 3)), np.ones(1, np.uint8), np.zeros((1, 3), np.uint8), -1)


def test_cutoff_band():
    s = np.array([0.3, 0.2, 0.2 * (1 + 3e-6), 0.1, 0.05])
    keep, band, drop = O.cutoff_band(s, 2)
    assert keep == {0} and band == {1, 2} and drop == {3, 4}
    assert O.kept_set_valid([0, 1], s, 2) and O.kept_set_valid([0, 2], s, 2)
    assert not O.kept_set_valid([1, 2], s, 2) and not O.kept_set_valid([0, 3], s, 2)
    keep, band, drop = O.cutoff_band(np.array([0.4, 0.3, 0.2]), 2)
    assert keep == {0, 1} and band == set() and drop == {2}


# ------------------------------------------------------------- compaction

def test_offsets_closed_form():
    kept = [np.array([0, 2]), np.array([], np.int64), np.array([1, 3, 4])]
    seg_idx, seg_off, tok_off = O.offsets(kept, 7, 3)
    assert list(seg_idx) == [0, 2, 1, 3, 4]
    assert list(seg_off) == [0, 2, 2, 5]
    assert list(tok_off) == [0, 5 * 7, 5 * 7 + 3 * 7, 5 * 7 + 3 * 7 + 6 * 7]


def test_keep_all_compaction_is_identity_copy():
    rng = np.random.default_rng(8)
    T, Fh, Fc = 5, 4, 2
    k = rng.standard_normal(((Fh + Fc) * T, 3, 8)).astype(np.float32)
    v = rng.standard_normal(((Fh + Fc) * T, 3, 8)).astype(np.float32)
    kept = [np.arange(Fh)] * 3
    k_c, v_c, _, _, tok_off = O.compact(k, v, kept, T, Fh, Fc)
    for h in range(3):
        assert np.array_equal(k_c[tok_off[h]:tok_off[h + 1]], k[:, h])
        assert np.array_equal(v_c[tok_off[h]:tok_off[h + 1]], v[:, h])


def test_compaction_rows_equal_boolean_frame_selection():
    rng = np.random.default_rng(9)
    T, Fh, Fc, H = 3, 6, 2, 3
    k = rng.integers(0, 65535, ((Fh + Fc) * T, H, 4)).astype(np.uint16)
    v = rng.integers(0, 65535, ((Fh + Fc) * T, H, 4)).astype(np.uint16)
    kept = [np.array([1, 4]), np.array([0, 2, 3, 5]), np.array([], np.int64)]
    k_c, v_c, _, _, tok_off = O.compact(k, v, kept, T, Fh, Fc)
    frame_of_token = np.arange((Fh + Fc) * T) // T
    for h in range(H):
        sel = np.isin(frame_of_token, np.concatenate([kept[h], np.arange(Fh, Fh + Fc)]))
        assert np.array_equal(k_c[tok_off[h]:tok_off[h + 1]], k[sel, h])
        assert np.array_equal(v_c[tok_off[h]:tok_off[h + 1]], v[sel, h])


# -------------------------------------------------------------- attention

def test_keep_all_reproduces_full_attention_exactly():
    rng = np.random.default_rng(10)
    T, Fh, Fc, D, H = 5, 4, 2, 16, 3
    q, k, v, _ = _rand_case(rng, H=H, D=D, T=T, Fh=Fh, Fc=Fc)
    role = np.array([0, 1, 0], np.uint8)
    mask = np.ones((H, Fh), np.uint8)
    c = O.compress(q, k, v, role, mask, Fh, T, Fh, Fc, 2)
    out = O.attend(q, c["k_c"], c["v_c"], c["tok_off"])
    dense = O.attend_dense(q, k, v)
    assert np.array_equal(out, dense)
    for h in range(H):
        np.testing.assert_allclose(dense[:, h], _sdpa(q[:, h], k[:, h], v[:, h], 1 / 4.0),
                                   rtol=0, atol=1e-12)


def test_compressed_attention_equals_library_on_selected_keys():
    rng = np.random.default_rng(11)
    T, Fh, Fc, D, H = 4, 6, 3, 16, 2
    q, k, v, role = _rand_case(rng, H=H, D=D, T=T, Fh=Fh, Fc=Fc)
    c = O.compress(q, k, v, role, np.zeros((H, Fh), np.uint8), 3, T, Fh, Fc, 2)
    out = O.attend(q, c["k_c"], c["v_c"], c["tok_off"])
    frame_of_token = np.arange((Fh + Fc) * T) // T
    for h in range(H):
        sel = np.isin(frame_of_token, list(c["kept"][h]) + list(range(Fh, Fh + Fc)))
        ref = _sdpa(q[:, h], k[sel, h], v[sel, h], 0.25)
        np.testing.assert_allclose(out[:, h], ref, rtol=0, atol=1e-12)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(12)
    T, Fh, Fc, D = 4, 3, 2, 8
    q, k, _, role = _rand_case(rng, H=2, D=D, T=T, Fh=Fh, Fc=Fc)
    v = np.full(k.shape, 0.625)
    c = O.compress(q, k, v, role, np.ones((2, Fh), np.uint8), 2, T, Fh, Fc, 1)
    out = O.attend(q, c["k_c"], c["v_c"], c["tok_off"])
    np.testing.assert_allclose(out, 0.625, rtol=0, atol=1e-14)


def test_single_key_output_is_that_value():
    rng = np.random.default_rng(13)
    D = 8
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((3, 1, D))
    v = rng.standard_normal((3, 1, D))
    # T=1, two history frames dropped (m=0, empty mask), one current frame
    c = O.compress(q, k, v, np.ones(1, np.uint8), np.zeros((1, 2), np.uint8), 0, 1, 2, 1, 1)
    assert c["k_c"].shape == (1, D)
    out = O.attend(q, c["k_c"], c["v_c"], c["tok_off"])
    np.testing.assert_allclose(out[0, 0], v[2, 0], rtol=0, atol=1e-15)


def test_zero_budget_and_empty_mask_attend_current_chunk_only():
    rng = np.random.default_rng(14)
    T, Fh, Fc, D = 5, 4, 2, 16
    q, k, v, _ = _rand_case(rng, H=2, D=D, T=T, Fh=Fh, Fc=Fc)
    role = np.array([0, 1], np.uint8)
    c = O.compress(q, k, v, role, np.zeros((2, Fh), np.uint8), 0, T, Fh, Fc, 2)
    out = O.attend(q, c["k_c"], c["v_c"], c["tok_off"])
    for h in range(2):
        ref = _sdpa(q[:, h], k[Fh * T:, h], v[Fh * T:, h], 0.25)
        np.testing.assert_allclose(out[:, h], ref, rtol=0, atol=1e-12)


def test_no_history_window():
    rng = np.random.default_rng(15)
    q, k, v, role = _rand_case(rng, H=2, D=8, T=3, Fh=0, Fc=2)
    c = O.compress(q, k, v, role, np.zeros((2, 0), np.uint8), 5, 3, 0, 2, 1)
    assert c["scores"].shape == (2, 0) and list(c["seg_off"]) == [0, 0, 0]
    np.testing.assert_allclose(O.attend(q, c["k_c"], c["v_c"], c["tok_off"]),
                               O.attend_dense(q, k, v), rtol=0, atol=1e-13)


def test_sampled_rows_match_full_rows():
    rng = np.random.default_rng(16)
    q, k, v, _ = _rand_case(rng, H=2, D=8, T=4, Fh=2, Fc=2)
    full = O.attend_dense(q, k, v, block=3)
    rows = np.array([5, 0, 7])
    np.testing.assert_array_equal(O.attend_dense(q, k, v, rows=rows), full[rows])


def test_bf16_decode_exact():
    vals = np.array([1.0, -2.5, 0.0078125, 3.140625, -0.0], np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(O.decode_bf16(bits), vals.astype(np.float64))


# --------------------------------------------------- randomized small shapes

@settings(max_examples=25, deadline=None)
@given(H=st.integers(1, 4), D=st.sampled_from([8, 16]), T=st.integers(1, 8),
       Fh=st.integers(0, 6), Fc=st.integers(1, 3), s=st.integers(1, 5),
       m=st.integers(0, 7), seed=st.integers(0, 2**31 - 1))
def test_hypothesis_pipeline_invariants(H, D, T, Fh, Fc, s, m, seed):
    rng = np.random.default_rng(seed)
    q, k, v, _ = _rand_case(rng, H=H, D=D, T=T, Fh=Fh, Fc=Fc)
    role = rng.integers(0, 2, H).astype(np.uint8)
    mask = rng.integers(0, 2, (H, Fh)).astype(np.uint8)
    c = O.compress(q, k, v, role, mask, m, T, Fh, Fc, s)
    for h in range(H):
        kh = c["kept"][h]
        assert list(kh) == sorted(set(kh))
        if role[h] == O.DYNAMIC:
            assert len(kh) == min(m, Fh)
            if Fh:
                assert list(kh) == _brute_force_topm(c["scores"][h], m)
                mass = O.frame_masses(q[:, h], k[:, h], T, s, O.logit_scale(D))
                np.testing.assert_allclose(mass.sum(axis=1), 1.0, atol=1e-12)
        else:
            assert list(kh) == list(np.flatnonzero(mask[h]))
        assert c["tok_off"][h + 1] - c["tok_off"][h] == (len(kh) + Fc) * T
    out = O.attend(q, c["k_c"], c["v_c"], c["tok_off"])
    frame_of_token = np.arange((Fh + Fc) * T) // T
    for h in range(H):
        sel = np.isin(frame_of_token, list(c["kept"][h]) + list(range(Fh, Fh + Fc)))
        ref = _sdpa(q[:, h], k[sel, h], v[sel, h], 1 / math.sqrt(D))
        np.testing.assert_allclose(out[:, h], ref, rtol=0, atol=1e-11)


# ------------------------------------------------ workload recipe vs pages

def test_static_mask_pattern_and_cache_reduction_golden():
    with open(os.path.join(GOLDEN, "workload_facts.json")) as f:
        g = json.load(f)
    for fh, frames in g["static_keep_frames"]["cases"].items():
        assert list(np.flatnonzero(W.chunk_boundary_mask(int(fh)))) == frames
    for name, t in g["tokens_per_latent_frame"]["cases"].items():
        assert W.WORKLOADS[name].tokens_per_frame == t
    # The 30-layer 480P recipe keeps about 70% of the history KV, the pages'
    # 30% cache reduction.
    w = W.WORKLOADS["480p_30layers"]
    kept = w.num_static * W.chunk_boundary_mask(w.hist_frames).sum() + \
        (w.num_heads - w.num_static) * min(w.budget_m, w.hist_frames)
    frac = kept / (w.num_heads * w.hist_frames)
    target = 1.0 - g["cache_reduction"]["value"]
    assert abs(frac - target) <= g["cache_reduction"]["tolerance"]
