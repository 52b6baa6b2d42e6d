"""GPU: the allocation-free compression entry point (fkv_compress_noalloc,
library-owned scratch memory) against fkv_compress with a caller workspace,
through the C ABI, on two calls in a row, the second on a smaller layer (the
scratch then holds the first call's contents)."""
import numpy as np
import pytest

from hybrid_kv_cache_amd import fkv
from hybrid_kv_cache_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.require_gpu()


def _results(ckv):
    n = ckv.kept_tokens
    return dict(k=fkv.to_host(ckv.k)[:n], v=fkv.to_host(ckv.v)[:n],
                tok_off=fkv.to_host(ckv.tok_off), seg_off=fkv.to_host(ckv.seg_off),
                seg_idx=fkv.to_host(ckv.seg_idx), seg_score=fkv.to_host(ckv.seg_score))


def _compare(w, inp):
    import torch
    desc = fkv.desc_for(w)
    q, k, v = G.upload(inp)
    role, mask = inp.head_role, inp.static_keep_mask
    ref = fkv.CompressedKV(desc, role, mask, w.budget_m)
    got = fkv.CompressedKV(desc, role, mask, w.budget_m)
    assert ref.workspace_bytes <= fkv.SCRATCH_BYTES
    G.announce(f"fkv_compress {w.name} H={w.num_heads} T={w.tokens_per_frame}")
    fkv.fkv_compress(desc, q, k, v, role, mask, w.budget_m, ref)
    G.announce(f"fkv_compress_noalloc {w.name} H={w.num_heads} T={w.tokens_per_frame}")
    fkv.fkv_compress_noalloc(desc, q, k, v, role, mask, w.budget_m, got)
    torch.cuda.synchronize()
    a, b = _results(ref), _results(got)
    H, Fh = w.num_heads, w.hist_frames
    for key in ("tok_off", "seg_off", "k", "v"):
        assert np.array_equal(a[key], b[key]), key
    n_idx = int(a["seg_off"][-1])
    assert np.array_equal(a["seg_idx"][:n_idx], b["seg_idx"][:n_idx])
    # scores: identical kernels in the same order, so identical bits (NaN for
    # static heads on both sides)
    sa, sb = a["seg_score"][: H * Fh], b["seg_score"][: H * Fh]
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))


def test_noalloc_matches_compress_twice_shrinking():
    big = W.WORKLOADS["480p_layer"]
    small = W.small_workload(tokens_per_frame=100, num_heads=3, hist_frames=6, budget_m=4,
                             num_static=1, seed=11)
    _compare(big, W.generate_layer(big, 0))
    _compare(small, W.generate_layer(small))
