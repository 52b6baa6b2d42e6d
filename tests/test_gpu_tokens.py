"""GPU parity of the token-granular variant (fkv_compress_tokens) against the
CPU oracle."""
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


def _check_candidates(gpu_pick, phi, budget, rel=1e-4):
    """The GPU's kept candidates (local indices) against the oracle's float64
    scores: every score clearly above the C-th best is kept, none clearly
    below, C in all (ties inside a band of rel * max |phi| may go either way;
    the GPU sums in fp32 in another order)."""
    n = len(phi)
    c = min(max(budget, 0), n)
    assert len(gpu_pick) == c and np.all(np.diff(gpu_pick) > 0)
    if c == 0 or c == n:
        assert np.array_equal(gpu_pick, np.arange(c))
        return 0
    order = np.lexsort((np.arange(n), -phi))
    cut = phi[order[c - 1]]
    eps = rel * max(np.abs(phi).max(), 1e-30)
    picked = np.zeros(n, dtype=bool)
    picked[gpu_pick] = True
    assert picked[phi > cut + eps].all(), "a clearly better candidate was dropped"
    assert not picked[phi < cut - eps].any(), "a clearly worse candidate was kept"
    return int(((phi >= cut - eps) & (phi <= cut + eps)).sum())


def run_tokens(w, inp, cfg, rows=None):
    import torch
    desc = fkv.desc_for(w)
    q, k, v = fkv.to_device(inp.q), fkv.to_device(inp.k), fkv.to_device(inp.v)
    ckv = fkv.CompressedKV(desc, inp.head_role, None, 0, token_cfg=cfg)
    src = torch.empty(max(ckv.kept_tokens, 1), dtype=torch.int32, device="cuda")
    G.announce(f"fkv_compress_tokens {w.name} T={w.tokens_per_frame} S={cfg.sink_frames} "
               f"R={cfg.recent_frames} C={cfg.budget_tokens} L={cfg.boundary_tokens}")
    fkv.fkv_compress_tokens(desc, cfg, q, k, v, inp.head_role, ckv, src)
    torch.cuda.synchronize()
    T, Fh, Fc = w.tokens_per_frame, w.hist_frames, w.cur_frames
    ref = O.compress_tokens(inp.q, inp.k, inp.v, inp.head_role, T, Fh, Fc, w.query_stride,
                            cfg.sink_frames, cfg.recent_frames, cfg.budget_tokens,
                            cfg.boundary_tokens)
    tok_off = fkv.to_host(ckv.tok_off)
    np.testing.assert_array_equal(tok_off, ref["tok_off"])
    n = int(tok_off[-1])
    gsrc = fkv.to_host(src)[:n].astype(np.int64)
    kc, vc = fkv.to_host(ckv.k)[:n], fkv.to_host(ckv.v)[:n]
    lo_c, hi_c = ref["cand"]
    band = 0
    for h in range(w.num_heads):
        a, b = int(tok_off[h]), int(tok_off[h + 1])
        s = gsrc[a:b]
        # the rows are the window rows the GPU's indices name
        assert np.array_equal(kc[a:b], inp.k[s, h]) and np.array_equal(vc[a:b], inp.v[s, h])
        if inp.head_role[h] == O.DYNAMIC:
            r = ref["src"][h]
            n_sink, n_rec = lo_c, w.hist_frames * T - hi_c
            assert np.array_equal(s[:n_sink], r[:n_sink])
            assert np.array_equal(s[len(s) - n_rec - Fc * T:], r[len(r) - n_rec - Fc * T:])
            pick = s[n_sink:len(s) - n_rec - Fc * T] - lo_c
            band += _check_candidates(pick, ref["phi"][h], cfg.budget_tokens)
        else:
            assert np.array_equal(s, ref["src"][h]), f"static head {h}"
    # attention over the GPU's cache, against the oracle over the same rows
    out = G.run_attend(desc, q, ckv, w.n_q, w.num_heads, w.head_dim, w.dtype)
    got = G.host_f64(out)
    if rows is not None:
        got = got[rows]
    want = O.attend(inp.q, kc, vc, tok_off, rows=rows)
    G.check_output(got, want, w.dtype)
    return band


@pytest.mark.parametrize("dtype,T,cfg,seed", [
    ("bf16", 100, (1, 3, 250, 20), 41),    # ragged tiles, all zones
    ("bf16", 37, (0, 0, 40, 0), 42),       # no sink or recent zone, sink-less static
    ("bf16", 50, (2, 1, 0, 80), 43),       # C = 0; end tokens cover whole chunks
    ("bf16", 64, (1, 2, 10 ** 6, 5), 44),  # C beyond the candidates: keep all
    ("f32", 40, (1, 2, 77, 7), 45),
])
def test_compress_tokens(dtype, T, cfg, seed):
    D = 128 if dtype == "bf16" else 64
    w = W.small_workload(name=f"tokens_{dtype}", dtype=dtype, head_dim=D, tokens_per_frame=T,
                         num_heads=5, hist_frames=9, num_static=2, query_stride=3, seed=seed)
    run_tokens(w, W.generate_layer(w), fkv.FkvTokenCfg(*cfg))


def test_compress_tokens_zero_queries_tie_to_lowest_index():
    """q = 0: every candidate scores exactly 0 on both sides, and the GPU keeps
    the C lowest-index candidates (the radix select's tie rule)."""
    w = W.small_workload(tokens_per_frame=30, num_heads=3, hist_frames=6, num_static=1, seed=46)
    inp = W.generate_layer(w, zero_q=True)
    band = run_tokens(w, inp, fkv.FkvTokenCfg(1, 1, 33, 4))
    assert band > 0   # every candidate sits in the tie band; the exact check is below
    import torch
    desc = fkv.desc_for(w)
    cfg = fkv.FkvTokenCfg(1, 1, 33, 4)
    ckv = fkv.CompressedKV(desc, inp.head_role, None, 0, token_cfg=cfg)
    src = torch.empty(ckv.kept_tokens, dtype=torch.int32, device="cuda")
    fkv.fkv_compress_tokens(desc, cfg, fkv.to_device(inp.q), fkv.to_device(inp.k),
                            fkv.to_device(inp.v), inp.head_role, ckv, src)
    torch.cuda.synchronize()
    s, off = fkv.to_host(src), fkv.to_host(ckv.tok_off)
    for h in range(w.num_heads):
        if inp.head_role[h] == O.DYNAMIC:
            row = s[off[h]:off[h + 1]]
            assert list(row[30:30 + 33]) == list(range(30, 63))


def test_compress_tokens_480p_shape():
    """The 480P window: sink frame, last chunk recent, 9 frames' worth of
    candidate tokens, half-frame chunk ends for static heads; attention on
    sampled rows."""
    w = W.WORKLOADS["480p_layer"]
    T = w.tokens_per_frame
    rows = np.random.default_rng(47).choice(w.n_q, 48, replace=False)
    run_tokens(w, W.generate_layer(w), fkv.FkvTokenCfg(1, 3, 9 * T, T // 2), rows=rows)
