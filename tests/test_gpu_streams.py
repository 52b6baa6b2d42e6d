"""GPU: stream ordering of fkv_compress, whose score-independent copies run on
a second stream inside the library (forked from the caller's stream before the
scoring, joined back before the dynamic heads' copies).  Compared bitwise with
the single-stream stage sequence of fkv_compress_timed on the same inputs:
  - on a caller stream whose previous kernels write the window (the copies must
    wait for them) and whose next kernels read the compressed cache (they must
    wait for the copies);
  - from two host threads on two streams at once, several layers each."""
import threading

import numpy as np
import pytest

from hybrid_kv_cache_amd import fkv
from hybrid_kv_cache_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.require_gpu()


def _host(w, ckv, k=None, v=None):
    """The written part of every output (seg_idx beyond seg_off[H] and the
    rows past kept_tokens are capacity, never written)."""
    n = ckv.kept_tokens
    seg_off = fkv.to_host(ckv.seg_off)
    return dict(k=fkv.to_host(ckv.k if k is None else k)[:n],
                v=fkv.to_host(ckv.v if v is None else v)[:n],
                tok_off=fkv.to_host(ckv.tok_off), seg_off=seg_off,
                seg_idx=fkv.to_host(ckv.seg_idx)[: int(seg_off[-1])],
                seg_score=fkv.to_host(ckv.seg_score)[: w.num_heads * w.hist_frames]
                .view(np.uint32))


def _serial(w, inp, q, k, v):
    """Scoring, selection and every copy on one stream, in that order."""
    desc = fkv.desc_for(w)
    ckv = fkv.CompressedKV(desc, inp.head_role, inp.static_keep_mask, w.budget_m)
    G.announce(f"fkv_compress_timed {w.name} layer={inp.layer}")
    fkv.fkv_compress_timed(desc, q, k, v, inp.head_role, inp.static_keep_mask, w.budget_m, ckv)
    return _host(w, ckv)


def _same(a, b, what):
    for key in a:
        assert np.array_equal(a[key], b[key]), f"{what}: {key}"


def test_compress_orders_against_caller_stream():
    import torch
    w = W.WORKLOADS["480p_layer"]
    inp = W.generate_layer(w, 0)
    q, k_src, v_src = G.upload(inp)
    ref = _serial(w, inp, q, k_src, v_src)
    desc = fkv.desc_for(w)
    k = torch.zeros_like(k_src)
    v = torch.zeros_like(v_src)
    ckv = fkv.CompressedKV(desc, inp.head_role, inp.static_keep_mask, w.budget_m)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    G.announce(f"fkv_compress {w.name} on a side stream after window writes")
    with torch.cuda.stream(s):
        # the window is written on the caller's stream right before the call,
        # and the compressed cache is read right after it
        k.copy_(k_src)
        v.copy_(v_src)
        fkv.fkv_compress(desc, q, k, v, inp.head_role, inp.static_keep_mask, w.budget_m, ckv,
                         stream=s)
        k_out = ckv.k.clone()
        v_out = ckv.v.clone()
    s.synchronize()
    torch.cuda.synchronize()
    _same(ref, _host(w, ckv, k_out, v_out), "caller stream")


def test_compress_from_two_threads_on_two_streams():
    import torch
    w = W.WORKLOADS["480p_30layers"]
    layers = [W.generate_layer(w, l) for l in range(4)]
    dev = [G.upload(inp) for inp in layers]
    refs = [_serial(w, inp, *d) for inp, d in zip(layers, dev)]
    desc = fkv.desc_for(w)
    reps = 3
    outs = {(t, r, l): fkv.CompressedKV(desc, layers[l].head_role, layers[l].static_keep_mask,
                                        w.budget_m)
            for t in range(2) for r in range(reps) for l in range(len(layers))}
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def worker(t):
        try:
            for r in range(reps):
                for l in range(len(layers)):
                    inp = layers[l]
                    q, k, v = dev[l]
                    fkv.fkv_compress(desc, q, k, v, inp.head_role, inp.static_keep_mask,
                                     w.budget_m, outs[(t, r, l)], stream=streams[t])
        except Exception as e:  # reported by the main thread
            errors.append(e)

    G.announce(f"fkv_compress {w.name} from 2 threads x {reps} x {len(layers)} layers")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    for st in streams:
        st.synchronize()
    torch.cuda.synchronize()
    assert not errors, errors
    for (t, r, l), ckv in outs.items():
        _same(refs[l], _host(w, ckv), f"thread {t} rep {r} layer {l}")


def test_compress_attend_from_two_threads_on_two_streams():
    """fkv_compress_attend (attention of the unscored heads on the side
    stream, three events per call) from two host threads at once: every
    cache and attention output equals the two-call result."""
    import torch
    w = W.WORKLOADS["480p_30layers"]
    layers = [W.generate_layer(w, l) for l in range(3)]
    dev = [G.upload(inp) for inp in layers]
    desc = fkv.desc_for(w)
    refs, ref_out = [], []
    for inp, (q, k, v) in zip(layers, dev):
        ckv = fkv.CompressedKV(desc, inp.head_role, inp.static_keep_mask, w.budget_m)
        out = torch.empty((w.n_q, w.num_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        fkv.fkv_compress(desc, q, k, v, inp.head_role, inp.static_keep_mask, w.budget_m, ckv)
        fkv.fkv_attend(desc, q, ckv, out, None)
        torch.cuda.synchronize()
        refs.append(_host(w, ckv))
        ref_out.append(fkv.to_host(out).view(np.uint16).copy())
    reps = 3
    outs = {}
    for t in range(2):
        for r in range(reps):
            for l, inp in enumerate(layers):
                outs[(t, r, l)] = (
                    fkv.CompressedKV(desc, inp.head_role, inp.static_keep_mask, w.budget_m),
                    torch.empty((w.n_q, w.num_heads, w.head_dim), dtype=torch.bfloat16,
                                device="cuda"))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def worker(t):
        try:
            for r in range(reps):
                for l, inp in enumerate(layers):
                    q, k, v = dev[l]
                    ckv, out = outs[(t, r, l)]
                    fkv.fkv_compress_attend(desc, q, k, v, inp.head_role, inp.static_keep_mask,
                                            w.budget_m, ckv, out, None, stream=streams[t])
        except Exception as e:  # reported by the main thread
            errors.append(e)

    G.announce(f"fkv_compress_attend {w.name} from 2 threads x {reps} x {len(layers)} layers")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    for st in streams:
        st.synchronize()
    torch.cuda.synchronize()
    assert not errors, errors
    for (t, r, l), (ckv, out) in outs.items():
        _same(refs[l], _host(w, ckv), f"thread {t} rep {r} layer {l}")
        assert np.array_equal(ref_out[l], fkv.to_host(out).view(np.uint16)), \
            f"attention output, thread {t} rep {r} layer {l}"
