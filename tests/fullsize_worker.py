"""Host side of the full-size parity tests, run in worker processes: one
layer's inputs (the seeded generator) and everything the oracle expects of
it.  Kept free of module-level NumPy so that a worker can cap its BLAS
threads before NumPy loads (several workers share the host's cores)."""
import os


def init_worker(blas_threads: int) -> None:
    for var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = str(blas_threads)


def sample_rows(w, layer, n_rows):
    import numpy as np
    rows = np.sort(np.random.default_rng(1000 + layer).choice(w.n_q, n_rows, replace=False))
    rows[0], rows[-1] = 0, w.n_q - 1
    return rows


def digest(a) -> str:
    """128-bit digest of an array's bytes (bitwise comparison of large
    compacted caches without shipping them between processes)."""
    import numpy as np
    import xxhash
    return xxhash.xxh3_128_hexdigest(np.ascontiguousarray(a).view(np.uint8))


def layer_job(name: str, layer: int, n_rows: int, with_dense: bool) -> dict:
    from hybrid_kv_cache_amd import workloads as W
    from oracle import forcing_kv as O
    w = W.WORKLOADS[name]
    inp = W.generate_layer(w, layer)
    role, mask = inp.head_role, inp.static_keep_mask
    scores = O.segment_scores(inp.q, inp.k, role, w.tokens_per_frame, w.hist_frames,
                              w.query_stride)
    kept = O.select_frames(scores, role, mask, w.budget_m)
    k_c, v_c, _, _, tok_off = O.compact(inp.k, inp.v, kept, w.tokens_per_frame,
                                        w.hist_frames, w.cur_frames)
    rows = sample_rows(w, layer, n_rows)
    ref = O.attend(inp.q, k_c, v_c, tok_off, rows=rows)
    dref = O.attend_dense(inp.q, inp.k, inp.v, rows=rows[::4]) if with_dense else None
    return dict(inp=inp, scores=scores, kept=kept, tok_off=tok_off, k_digest=digest(k_c),
                v_digest=digest(v_c), rows=rows, ref=ref, dref=dref)
