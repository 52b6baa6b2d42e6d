"""Pins of the oracle's head-profiling functions, and the library's host
classifier against them (CPU only)."""
import numpy as np
import pytest
import torch

from hybrid_kv_cache_amd import fkv
from hybrid_kv_cache_amd import workloads as W
from oracle import forcing_kv as O


def test_profile_masses_match_sdpa_frame_indicators():
    """Mean mass per frame = attention (torch SDPA, float64) with one-hot frame
    indicators as values, averaged over the sampled queries; rows sum to 1."""
    w = W.small_workload(dtype="f32", head_dim=64, tokens_per_frame=7, num_heads=3,
                         hist_frames=6, seed=21)
    inp = W.generate_layer(w)
    T, s = w.tokens_per_frame, 2
    m = O.profile_masses(inp.q, inp.k, T, s)
    np.testing.assert_allclose(m.sum(axis=1), 1.0, rtol=1e-12)
    F = w.frames
    ind = np.kron(np.eye(F), np.ones((T, 1)))            # [N_win, F]
    rows = np.arange(0, w.n_q, s)
    for h in range(w.num_heads):
        qh = torch.tensor(inp.q[rows, h], dtype=torch.float64)[None]
        kh = torch.tensor(inp.k[:, h], dtype=torch.float64)[None]
        vh = torch.tensor(ind, dtype=torch.float64)[None]
        att = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh)[0].numpy()
        np.testing.assert_allclose(m[h], att.mean(axis=0), rtol=1e-10, atol=1e-14)


def test_chunk_discontinuity_closed_forms():
    # boundary frames of 6 with F_c = 3: 0, 2, 3, 5; inner 1, 4
    assert O.chunk_discontinuity(np.full(6, 1 / 6), 3) == pytest.approx(1.0)
    assert O.chunk_discontinuity(np.array([.2, .1, .2, .2, .1, .2]), 3) == pytest.approx(2.0)
    assert np.isnan(O.chunk_discontinuity(np.array([.25, 0, .25, .25, 0, .25]), 3))
    assert np.isnan(O.chunk_discontinuity(np.full(4, .25), 2))   # every frame a boundary
    # reversed preference: inner frames heavier
    assert O.chunk_discontinuity(np.array([.1, .2, .1, .1, .4, .1]), 3) == pytest.approx(1 / 3)


def test_classify_heads_rule():
    mass = np.array([[.2, .1, .2, .2, .1, .2, 0, 0, 0],
                     [1 / 9] * 9,
                     [.25, 0, .25, .25, 0, .25, 0, 0, 0]]) * 3     # summed over 3 calls
    role, mask, disc = O.classify_heads(mass, 3, 6, 3, 1.5)
    assert list(role) == [O.STATIC, O.DYNAMIC, O.DYNAMIC]         # NaN -> dynamic
    assert list(mask[0]) == [1, 0, 1, 1, 0, 1]                    # >= 1/9 of the mass
    assert not mask[1].any() and not mask[2].any()
    np.testing.assert_allclose(disc[:2], [2.0, 1.0])


def test_planted_static_heads_are_recovered():
    """The profiling sample plants a boundary signature on the heads the
    generator draws static: the oracle's labels recover exactly those."""
    w = W.small_workload(tokens_per_frame=20, num_heads=6, hist_frames=9, num_static=3, seed=22)
    total = None
    for sample in range(2):
        inp = W.generate_profile_sample(w, sample)
        m = O.profile_masses(inp.q, inp.k, w.tokens_per_frame, 1)
        total = m if total is None else total + m
    role, mask, disc = O.classify_heads(total, 2, w.hist_frames, w.cur_frames, 2.0)
    truth = W.generate_profile_sample(w, 1).head_role
    assert np.array_equal(truth, W.generate_layer(w, 0).head_role)   # roles of the model
    assert np.array_equal(role, truth)
    assert (disc[truth == O.STATIC] > 2.5).all() and (disc[truth == O.DYNAMIC] < 1.5).all()


def test_library_classifier_matches_oracle():
    """fkv_classify_heads (host C) against the oracle on random summed masses,
    including exact-threshold and degenerate rows."""
    fkv.load()
    rng = np.random.default_rng(23)
    for trial in range(200):
        H, Fh, Fc = int(rng.integers(1, 9)), int(rng.integers(0, 13)), int(rng.integers(1, 5))
        Ft = Fh + Fc
        mass = rng.random((H, Ft)).astype(np.float32)
        mass[rng.random((H, Ft)) < 0.3] = 0
        n = int(rng.integers(1, 4))
        thr = float(rng.choice([0.5, 1.0, 1.5, 2.0]))
        d = fkv.make_desc(H, 128, 4, Fh, Fc, 1)
        role, mask, disc = fkv.fkv_classify_heads(d, mass, n, thr)
        r2, m2, d2 = O.classify_heads(mass.astype(np.float64), n, Fh, Fc, thr)
        np.testing.assert_allclose(disc, d2, rtol=1e-6, equal_nan=True)
        ok = ~np.isclose(d2, thr, rtol=1e-6)          # decisions away from a tie
        assert np.array_equal(role[ok], r2[ok]), trial
        assert np.array_equal(mask[ok], m2[ok]), trial
