"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: kept frames and offsets against the oracle (up to the
cutoff tie band), the compacted K/V bitwise, and the attention output on a
seeded sample of query rows that the oracle computes one by one."""
import numpy as np
import pytest

from hybrid_kv_cache_amd import fkv
from hybrid_kv_cache_amd import workloads as W
from oracle import forcing_kv as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

ROW_SAMPLE = 96


@pytest.fixture(autouse=True)
def _gpu():
    G.require_gpu()


def check_layer(w, layer):
    inp = W.generate_layer(w, layer)
    role, mask = inp.head_role, inp.static_keep_mask
    desc, ckv, (q, k, v), res = G.run_compress(w, inp)
    scores = O.segment_scores(inp.q, inp.k, role, w.tokens_per_frame, w.hist_frames,
                              w.query_stride)
    G.check_scores(res, scores, role)
    kept = G.check_selection(w, res, scores, role, mask, w.budget_m)
    k_c, v_c, _, _, tok_off = O.compact(inp.k, inp.v, kept, w.tokens_per_frame,
                                        w.hist_frames, w.cur_frames)
    n = int(tok_off[-1])
    assert np.array_equal(fkv.to_host(ckv.k)[:n], k_c), "compacted K differs"
    assert np.array_equal(fkv.to_host(ckv.v)[:n], v_c), "compacted V differs"
    out = G.run_attend(desc, q, ckv, w.n_q, w.num_heads, w.head_dim, w.dtype)
    rows = np.sort(np.random.default_rng(1000 + layer).choice(w.n_q, ROW_SAMPLE, replace=False))
    rows[0], rows[-1] = 0, w.n_q - 1
    ref = O.attend(inp.q, k_c, v_c, tok_off, rows=rows)
    got = G.host_f64(out)[rows]
    G.check_output(got, ref, w.dtype)
    dout = G.run_attend_dense(desc, q, k, v, w.n_q, w.num_heads, w.head_dim, w.dtype)
    dref = O.attend_dense(inp.q, inp.k, inp.v, rows=rows[::4])
    G.check_output(G.host_f64(dout)[rows[::4]], dref, w.dtype)


def test_480p_layer():
    check_layer(W.WORKLOADS["480p_layer"], 0)


@pytest.mark.parametrize("layer", range(30))
def test_480p_30layers(layer):
    """Every layer of the 30-layer 480P pass (own seed, head roles, masks)."""
    check_layer(W.WORKLOADS["480p_30layers"], layer)


def test_1080p_layer():
    check_layer(W.WORKLOADS["1080p_layer"], 0)


def test_720p_14b_layer0():
    check_layer(W.WORKLOADS["720p_14b_40layers"], 0)
