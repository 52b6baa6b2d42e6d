"""Pins of the oracle's token-granular functions (static_token_keep,
participative_scores, select_top_tokens, compress_tokens)."""
import numpy as np
import pytest

from hybrid_kv_cache_amd import workloads as W
from oracle import forcing_kv as O


def test_static_token_keep_closed_forms():
    T, Fh, Fc = 10, 6, 3
    # boundary_tokens = T keeps whole first and last frames: the frame-level
    # pattern (sink + chunk boundary frames) expanded to tokens
    frames = np.flatnonzero(W.chunk_boundary_mask(Fh, Fc))
    want = np.concatenate([np.arange(f * T, (f + 1) * T) for f in frames])
    assert np.array_equal(O.static_token_keep(Fh, T, Fc, 1, T), want)
    # no boundary tokens: the sink frames only
    assert np.array_equal(O.static_token_keep(Fh, T, Fc, 2, 0), np.arange(2 * T))
    # half a chunk or more from each end: every history token
    assert np.array_equal(O.static_token_keep(Fh, T, Fc, 0, 15), np.arange(Fh * T))
    # a trailing partial chunk keeps its own two ends
    assert list(O.static_token_keep(4, 5, 3, 0, 1)) == [0, 14, 15, 19]
    # counts at the 480P shape: sink frame + 780 tokens at each end of 6 chunks
    assert len(O.static_token_keep(18, 1560, 3, 1, 780)) == 1560 + 780 + 5 * 1560


def test_select_top_tokens_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(300):
        n = int(rng.integers(0, 40))
        phi = rng.integers(-3, 4, n).astype(np.float64)        # many ties
        c = int(rng.integers(-1, n + 3))
        got = O.select_top_tokens(phi, c)
        order = np.lexsort((np.arange(n), -phi))              # phi desc, index asc
        want = np.sort(order[:min(max(c, 0), n)])
        assert np.array_equal(got, want), (phi, c)


def test_participative_scores_properties():
    w = W.small_workload(dtype="f32", head_dim=64, tokens_per_frame=8, num_heads=2,
                         hist_frames=5, seed=4)
    inp = W.generate_layer(w)
    q, k = inp.q[:, 0], inp.k[:, 0]
    p = O.participative_scores(q, k, 3)
    rows = np.arange(0, w.n_q, 3)
    # one dot product per (sampled query, token), summed: the mean query times k
    np.testing.assert_allclose(p, k.astype(np.float64) @ q[rows].astype(np.float64).sum(0),
                               rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(O.participative_scores(2 * q, k, 3), 2 * p, rtol=1e-12)
    # q = 0: every score 0, the first C candidates are kept
    z = O.participative_scores(np.zeros_like(q), k, 3)
    assert not z.any() and list(O.select_top_tokens(z, 4)) == [0, 1, 2, 3]
    # a key along the summed query ranks first
    kk = k.copy()
    kk[17] = q[rows].sum(0) / np.linalg.norm(q[rows].sum(0)) * 50
    assert O.select_top_tokens(O.participative_scores(q, kk, 3), 1)[0] == 17


def test_compress_tokens_structure():
    w = W.small_workload(tokens_per_frame=10, num_heads=4, hist_frames=9, num_static=2,
                         query_stride=2, seed=5)
    inp = W.generate_layer(w)
    T, Fh, Fc = 10, 9, 3
    S, R, C, L = 1, 3, 25, 3
    r = O.compress_tokens(inp.q, inp.k, inp.v, inp.head_role, T, Fh, Fc, 2, S, R, C, L)
    assert r["cand"] == (S * T, (Fh - R) * T)
    for h in range(4):
        src = r["src"][h]
        assert np.all(np.diff(src) > 0)
        assert np.array_equal(src[-Fc * T:], np.arange(Fh * T, (Fh + Fc) * T))
        lo, hi = r["tok_off"][h], r["tok_off"][h + 1]
        assert np.array_equal(r["k_c"][lo:hi], inp.k[src, h])
        assert np.array_equal(r["v_c"][lo:hi], inp.v[src, h])
        if inp.head_role[h] == O.DYNAMIC:
            hist = src[:-Fc * T]
            assert len(hist) == S * T + C + R * T
            assert np.array_equal(hist[:S * T], np.arange(S * T))
            assert np.array_equal(hist[-R * T:], np.arange((Fh - R) * T, Fh * T))
            picked = hist[S * T:-R * T] - S * T
            assert np.array_equal(picked, O.select_top_tokens(r["phi"][h], C))
        else:
            assert np.array_equal(src[:-Fc * T], O.static_token_keep(Fh, T, Fc, S, L))


def test_compress_tokens_keep_all_equals_frame_level_keep_all():
    """Budget covering every candidate and static ends covering whole chunks:
    every head keeps the whole window, as the frame-level path does with
    m = F_h and an all-ones mask."""
    w = W.small_workload(tokens_per_frame=6, num_heads=3, hist_frames=6, num_static=1, seed=6)
    inp = W.generate_layer(w)
    T, Fh, Fc = 6, 6, 3
    r = O.compress_tokens(inp.q, inp.k, inp.v, inp.head_role, T, Fh, Fc, 4, 1, 2, 10 ** 6, 9)
    f = O.compress(inp.q, inp.k, inp.v, inp.head_role, np.ones((3, Fh), np.uint8), Fh, T, Fh,
                   Fc, 4)
    assert np.array_equal(r["tok_off"], f["tok_off"])
    assert np.array_equal(r["k_c"], f["k_c"]) and np.array_equal(r["v_c"], f["v_c"])
