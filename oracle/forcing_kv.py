"""CPU oracle for the Forcing-KV hybrid head-wise KV-cache compression path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  It shares no
code with the HIP library (``hybrid_kv_cache_amd``) and neither side imports
the other; the seeded input generator is the only thing both use.

Everything here is plain NumPy in float64, written step by step in the order
the method takes them, with no blocking, fusion or reordering beyond what the
definitions state.  Sources (pages on the method):

  [S] "Forcing-KV：面向高效自回归视频扩散模型的混合KV缓存压缩" (ai-feeds.com
      summary of arXiv 2605.09681), section 方法 (Method):
        › 输入与整体流程 (input and overall flow)   -> per-layer, per-frame cache
        › 关键模块 › 2 静态结构剪枝 (static structural pruning) -> select_static
        › 关键模块 › 3 动态相似性剪枝 (dynamic similarity pruning) -> scoring,
          select_dynamic
        › 输出与工程收益 (output)  -> compact, attend
  [A] "Forcing-KV: Hybrid KV Cache Compression for Efficient Autoregressive
      Video Diffusion Models" (tomesphere.com), Abstract: static heads get
      structured static pruning, dynamic heads get pruning by segment-wise
      similarity.

Where the pages leave a step open, the reading taken is stated at the function
(scoring rule: softmax attention mass per frame from a strided sample of the
current chunk's queries, over the whole window including the current chunk;
ranking ties broken by the lower frame index; kept frames in ascending order,
the current chunk last; non-causal attention with scale 1/sqrt(D)).

Pinned by tests/test_oracle_pins.py (invariants, closed forms, brute force,
library cross-checks); for the rolling cache by tests/test_oracle_rolling.py
(reduction to the plain window, recomputation from the frame store); for the
e4m3 cache by tests/test_oracle_fp8.py (hand-decoded codes, exactly
representable inputs with power-of-two head scales); for the token variant by
tests/test_oracle_tokens.py; for head profiling by
tests/test_oracle_profile.py.  Parity of generic numeric outputs is otherwise
pinned only through those checks; no page prints a worked example.

Layouts (token-major):  q [Nq, H, D];  k, v [N_win, H, D] with the window's
frames oldest first and the current chunk's ``F_c`` frames last.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

STATIC = 0
DYNAMIC = 1
TIE_REL = 1e-5


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    """Inputs come as float32 values or bf16 bit patterns; both convert exactly."""
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return np.asarray(x, dtype=np.float64)


def logit_scale(head_dim: int, scale: float = 0.0) -> float:
    """Softmax temperature: 1/sqrt(D) unless the caller gives one (the pages
    are silent; standard scaled dot-product attention is assumed)."""
    return float(scale) if scale else 1.0 / math.sqrt(head_dim)


def sampled_query_rows(n_q: int, stride: int) -> np.ndarray:
    """The strided query sample used for scoring: rows 0, s, 2s, ... < Nq."""
    return np.arange(0, n_q, stride, dtype=np.int64)


def frame_masses(q_h: np.ndarray, k_h: np.ndarray, tokens_per_frame: int,
                 stride: int, scale: float) -> np.ndarray:
    """Attention mass each window frame receives from each sampled query of one
    head.  [S] 关键模块 › 3: the history cache is grouped by frame and each group
    is scored by attention against the current queries.

    q_h [Nq, D], k_h [N_win, D] in float64.  For each sampled query i:
      z_j = scale * q_i . k_j            for every window key j
      p   = softmax(z)                   over the WHOLE window (history and
                                         the current chunk alike)
      mass[i, f] = sum of p_j over the T tokens of frame f
    Returns mass [n_s, F_total].
    """
    rows = sampled_query_rows(q_h.shape[0], stride)
    n_win = k_h.shape[0]
    n_frames = n_win // tokens_per_frame
    # the steps below work in place on one [n_s, N_win] array (the same
    # operations in the same order as z = scale * q k^T; z -= max; p = e^z /
    # sum e^z), to keep memory and time down at the largest window sizes
    z = q_h[rows] @ k_h.T
    z *= scale
    z -= z.max(axis=1, keepdims=True)
    np.exp(z, out=z)
    z /= z.sum(axis=1, keepdims=True)
    return z.reshape(len(rows), n_frames, tokens_per_frame).sum(axis=2)


def segment_scores(q: np.ndarray, k: np.ndarray, head_role: np.ndarray,
                   tokens_per_frame: int, hist_frames: int, stride: int,
                   scale: float = 0.0) -> np.ndarray:
    """Per-head score of every history frame.  [S] 关键模块 › 3.

    Dynamic head h: score[h, f] = mean over the sampled queries of mass[i, f],
    for the history frames f < F_h.  Static heads are not scored (NaN).
    """
    q = as_f64(q)
    k = as_f64(k)
    H, D = q.shape[1], q.shape[2]
    sc = logit_scale(D, scale)
    out = np.full((H, hist_frames), np.nan, dtype=np.float64)
    for h in range(H):
        if head_role[h] != DYNAMIC or hist_frames == 0:
            continue
        mass = frame_masses(q[:, h, :], k[:, h, :], tokens_per_frame, stride, sc)
        out[h] = mass[:, :hist_frames].mean(axis=0)
    return out


def select_static(mask_row: np.ndarray) -> np.ndarray:
    """[S] 关键模块 › 2: a static head keeps the fixed, profiled positions,
    taken by mask.  Frame granular: the kept history frames are those whose
    mask entry is set, in ascending order."""
    return np.flatnonzero(np.asarray(mask_row) != 0).astype(np.int64)


def select_dynamic(score_row: np.ndarray, budget_m: int) -> np.ndarray:
    """[S] 关键模块 › 3: keep the few best-scoring frames.  The m_eff = min(m, F_h)
    frames ranked first by (score descending, frame index ascending), returned
    in ascending frame order."""
    f_h = len(score_row)
    m_eff = min(budget_m, f_h)
    order = sorted(range(f_h), key=lambda f: (-score_row[f], f))
    return np.array(sorted(order[:m_eff]), dtype=np.int64)


def select_frames(scores: np.ndarray, head_role: np.ndarray,
                  static_keep_mask: np.ndarray, budget_m: int) -> List[np.ndarray]:
    """Kept history frames per head ([A]: static heads by structure, dynamic
    heads by segment similarity)."""
    if budget_m < 0:
        raise ValueError("budget_m must be >= 0")
    kept = []
    for h in range(len(head_role)):
        if head_role[h] == DYNAMIC:
            kept.append(select_dynamic(scores[h], budget_m))
        else:
            kept.append(select_static(static_keep_mask[h]))
    return kept


def offsets(kept: Sequence[np.ndarray], tokens_per_frame: int, cur_frames: int):
    """Ragged layout bookkeeping.  seg_idx = the kept history frames of head 0,
    then head 1, ...; seg_off[h] = where head h's frames start in seg_idx;
    tok_off[h] = first compacted row of head h, each head holding its kept
    history frames followed by the current chunk."""
    H = len(kept)
    seg_off = np.zeros(H + 1, dtype=np.int64)
    tok_off = np.zeros(H + 1, dtype=np.int64)
    for h in range(H):
        seg_off[h + 1] = seg_off[h] + len(kept[h])
        tok_off[h + 1] = tok_off[h] + (len(kept[h]) + cur_frames) * tokens_per_frame
    seg_idx = (np.concatenate(kept) if H and seg_off[H] else np.zeros(0)).astype(np.int64)
    return seg_idx, seg_off, tok_off


def compact(k: np.ndarray, v: np.ndarray, kept: Sequence[np.ndarray],
            tokens_per_frame: int, hist_frames: int, cur_frames: int):
    """[S] 输出与工程收益: the compressed K/V that replace the cache in attention.

    Head-major ragged rows: for head h, the T rows of each kept history frame
    (ascending), then the T rows of each current-chunk frame.  A pure copy:
    values are returned in the input's own dtype, unchanged.
    Returns k_c, v_c [tok_off[H], D] and the offsets.
    """
    T = tokens_per_frame
    seg_idx, seg_off, tok_off = offsets(kept, T, cur_frames)
    H, D = k.shape[1], k.shape[2]
    k_c = np.empty((int(tok_off[H]), D), dtype=k.dtype)
    v_c = np.empty((int(tok_off[H]), D), dtype=v.dtype)
    for h in range(H):
        frames = list(kept[h]) + list(range(hist_frames, hist_frames + cur_frames))
        row = int(tok_off[h])
        for f in frames:
            k_c[row:row + T] = k[f * T:(f + 1) * T, h, :]
            v_c[row:row + T] = v[f * T:(f + 1) * T, h, :]
            row += T
    return k_c, v_c, seg_idx, seg_off, tok_off


def softmax_attention(q_rows: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                      scale: float) -> np.ndarray:
    """Textbook attention of a block of queries over a set of keys, float64:
    softmax(scale * q k^T) v, non-causal."""
    z = (q_rows @ k_rows.T) * scale
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)) @ v_rows


def attend(q: np.ndarray, k_c: np.ndarray, v_c: np.ndarray, tok_off: np.ndarray,
           scale: float = 0.0, rows: Optional[np.ndarray] = None,
           block: int = 1024) -> np.ndarray:
    """[S] 输出与工程收益: the current chunk's queries attend over the compressed
    cache.  Every query of head h sees all of head h's compacted rows (kept
    history frames and the current chunk); no causal mask inside the window.

    rows: optional subset of query indices (for large cases); returns
    [len(rows) or Nq, H, D] float64.
    """
    qf = as_f64(q)
    H, D = qf.shape[1], qf.shape[2]
    sc = logit_scale(D, scale)
    sel = np.arange(qf.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((len(sel), H, D), dtype=np.float64)
    for h in range(H):
        lo, hi = int(tok_off[h]), int(tok_off[h + 1])
        kc, vc = as_f64(k_c[lo:hi]), as_f64(v_c[lo:hi])   # this head's rows, exact
        for b in range(0, len(sel), block):
            r = sel[b:b + block]
            out[b:b + block, h] = softmax_attention(qf[r, h], kc, vc, sc)
    return out


def attend_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float = 0.0,
                 rows: Optional[np.ndarray] = None, block: int = 1024) -> np.ndarray:
    """Full-KV baseline: every query attends over the whole uncompressed window."""
    qf = as_f64(q)
    H, D = qf.shape[1], qf.shape[2]
    sc = logit_scale(D, scale)
    sel = np.arange(qf.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((len(sel), H, D), dtype=np.float64)
    for h in range(H):
        kf, vf = as_f64(k[:, h]), as_f64(v[:, h])           # this head's keys, exact
        for b in range(0, len(sel), block):
            r = sel[b:b + block]
            out[b:b + block, h] = softmax_attention(qf[r, h], kf, vf, sc)
    return out


def compress(q, k, v, head_role, static_keep_mask, budget_m: int,
             tokens_per_frame: int, hist_frames: int, cur_frames: int,
             query_stride: int, scale: float = 0.0) -> Dict[str, np.ndarray]:
    """The whole compression step of one layer: score, select, compact."""
    scores = segment_scores(q, k, head_role, tokens_per_frame, hist_frames,
                            query_stride, scale)
    kept = select_frames(scores, head_role, static_keep_mask, budget_m)
    k_c, v_c, seg_idx, seg_off, tok_off = compact(k, v, kept, tokens_per_frame,
                                                  hist_frames, cur_frames)
    return dict(scores=scores, kept=kept, k_c=k_c, v_c=v_c, seg_idx=seg_idx,
                seg_off=seg_off, tok_off=tok_off)


def compress_ragged(q, hist_k, hist_v, hist_tok_off, cur_k, cur_v, head_role,
                    static_keep_mask, budget_m: int, tokens_per_frame: int,
                    cur_frames: int, query_stride: int, scale: float = 0.0
                    ) -> Dict[str, np.ndarray]:
    """Compression of one layer whose history differs from head to head (a
    rolling compressed cache, [S] 输出与工程收益: the compressed K/V replace the
    cache, here also for the next chunk).

    Head h's window is its own history, the T-row frames of rows
    [hist_tok_off[h], hist_tok_off[h+1]) of hist_k / hist_v (oldest first),
    followed by the current chunk's frames cur_k[:, h] ([F_c T, H, D]).
    Scoring, selection and compaction follow compress() head by head, with
    F_h replaced by the head's own history length n_h: a dynamic head scores
    its n_h history frames by the mean softmax mass over its whole window and
    keeps min(m, n_h); a static head keeps the frames its mask row marks among
    its n_h (mask entries beyond n_h must be 0).  scores [H, F_h max] hold NaN
    beyond n_h and for static heads.
    """
    T = tokens_per_frame
    qf = as_f64(q)
    H, D = qf.shape[1], qf.shape[2]
    sc = logit_scale(D, scale)
    f_max = static_keep_mask.shape[1]
    if budget_m < 0:
        raise ValueError("budget_m must be >= 0")
    scores = np.full((H, f_max), np.nan, dtype=np.float64)
    kept = []
    n_hist = []
    for h in range(H):
        lo, hi = int(hist_tok_off[h]), int(hist_tok_off[h + 1])
        if (hi - lo) % T:
            raise ValueError("a history range is not a whole number of frames")
        n_h = (hi - lo) // T
        if n_h > f_max:
            raise ValueError("a head's history is longer than the mask rows")
        n_hist.append(n_h)
        if head_role[h] == DYNAMIC:
            if n_h:
                win = np.concatenate([as_f64(hist_k[lo:hi]), as_f64(cur_k[:, h])], axis=0)
                mass = frame_masses(qf[:, h, :], win, T, query_stride, sc)
                scores[h, :n_h] = mass[:, :n_h].mean(axis=0)
            kept.append(select_dynamic(scores[h, :n_h], budget_m))
        else:
            if np.any(np.asarray(static_keep_mask[h, n_h:]) != 0):
                raise ValueError("static mask marks a frame beyond the head's history")
            kept.append(select_static(static_keep_mask[h, :n_h]))
    seg_idx, seg_off, tok_off = offsets(kept, T, cur_frames)
    k_c = np.empty((int(tok_off[H]), D), dtype=hist_k.dtype)
    v_c = np.empty((int(tok_off[H]), D), dtype=hist_v.dtype)
    for h in range(H):
        lo = int(hist_tok_off[h])
        row = int(tok_off[h])
        for f in kept[h]:
            k_c[row:row + T] = hist_k[lo + f * T:lo + (f + 1) * T]
            v_c[row:row + T] = hist_v[lo + f * T:lo + (f + 1) * T]
            row += T
        for j in range(cur_frames):
            k_c[row:row + T] = cur_k[j * T:(j + 1) * T, h, :]
            v_c[row:row + T] = cur_v[j * T:(j + 1) * T, h, :]
            row += T
    return dict(scores=scores, kept=kept, n_hist=np.array(n_hist), k_c=k_c, v_c=v_c,
                seg_idx=seg_idx, seg_off=seg_off, tok_off=tok_off)


def refresh_current(k_c, v_c, tok_off, cur_k, cur_v, tokens_per_frame: int,
                    cur_frames: int):
    """Selection reused across the denoising steps of one chunk: the kept
    history rows stay, and the last F_c frames of every head's range (its
    current chunk) are copied again from the new cur_k / cur_v [F_c T, H, D]."""
    T = tokens_per_frame
    k2, v2 = k_c.copy(), v_c.copy()
    for h in range(len(tok_off) - 1):
        hi = int(tok_off[h + 1])
        for j in range(cur_frames):
            r = hi - (cur_frames - j) * T
            k2[r:r + T] = cur_k[j * T:(j + 1) * T, h, :]
            v2[r:r + T] = cur_v[j * T:(j + 1) * T, h, :]
    return k2, v2


def is_chunk_boundary(frame_id: int, cur_frames: int) -> bool:
    """Frame ids count from 0, chunks are the aligned runs of F_c ids: a
    frame is a boundary when it is the sink (id 0) or the first or last frame
    of its chunk ([S] 关键模块 › 1 and 2: static heads attend to chunk start and
    end positions)."""
    return frame_id == 0 or frame_id % cur_frames in (0, cur_frames - 1)


def roll_static_keep(frame_ids: Sequence[int], cur_frames: int, cap: int) -> np.ndarray:
    """Static head in a rolling cache: keep the boundary frames of its history
    (ids as above); while more than cap are kept, drop the oldest kept frame
    that is not the sink.  Returns a 0/1 mask over frame_ids."""
    keep = [i for i, fid in enumerate(frame_ids) if is_chunk_boundary(int(fid), cur_frames)]
    while len(keep) > cap:
        drop = next((j for j, i in enumerate(keep) if frame_ids[i] != 0), 0)
        keep.pop(drop)
    mask = np.zeros(len(frame_ids), dtype=np.uint8)
    mask[keep] = 1
    return mask


def default_static_cap(hist_frames: int, cur_frames: int) -> int:
    """Kept-frame cap of static heads in a rolling cache: as many frames as the
    boundary pattern keeps in a plain window of F_h frames (the static
    reduction stays constant in size, [S] 关键模块 › 2), and never more than
    F_h - F_c, so that no history outgrows the window."""
    n = sum(1 for f in range(hist_frames) if is_chunk_boundary(f, cur_frames))
    return min(n, max(hist_frames - cur_frames, 0))


def rollout(q_chunks: Sequence[np.ndarray], k_all: np.ndarray, v_all: np.ndarray,
            head_role, budget_m: int, tokens_per_frame: int, hist_frames: int,
            cur_frames: int, query_stride: int, scale: float = 0.0,
            static_cap: Optional[int] = None) -> List[Dict]:
    """Consecutive chunk steps of one layer with a rolling compressed cache.

    Chunk 0 compresses the plain window (frames [0, F_h + F_c) of the frame
    store k_all / v_all).  The compressed cache of chunk c - 1 (kept history,
    then its now finished current chunk) is chunk c's history: frames not kept
    are gone for good, the finished chunk is appended.  Chunk c's current
    frames are [F_h + c F_c, F_h + (c + 1) F_c) of the store.  Static heads
    keep the boundary frames of their history (roll_static_keep, chunk 0
    included) up to static_cap (default_static_cap unless given, at most
    F_h - F_c so that no history outgrows F_h frames); dynamic heads keep
    their top m, which must also be at most F_h - F_c.
    Each result carries the static masks used (``mask`` [H, F_h]) and the
    absolute frame ids of every head's compacted frames (``ids``).
    """
    T, Fh, Fc = tokens_per_frame, hist_frames, cur_frames
    H = len(head_role)
    if budget_m > Fh - Fc:
        raise ValueError("a rolling cache needs m <= F_h - F_c")
    cap = default_static_cap(Fh, Fc) if static_cap is None else static_cap
    if cap > Fh - Fc:
        raise ValueError("a rolling cache needs static_cap <= F_h - F_c")
    out = []
    for c in range(len(q_chunks)):
        first = Fh + c * Fc
        prev_ids = [list(range(Fh))] * H if c == 0 else out[-1]["ids"]
        mask = np.zeros((H, Fh), dtype=np.uint8)
        for h in range(H):
            if head_role[h] != DYNAMIC:
                mk = roll_static_keep(prev_ids[h], Fc, cap)
                mask[h, :len(mk)] = mk
        if c == 0:
            n_win = (Fh + Fc) * T
            r = compress(q_chunks[0], k_all[:n_win], v_all[:n_win], head_role, mask,
                         budget_m, T, Fh, Fc, query_stride, scale)
        else:
            prev = out[-1]
            cur_k = k_all[first * T:(first + Fc) * T]
            cur_v = v_all[first * T:(first + Fc) * T]
            r = compress_ragged(q_chunks[c], prev["k_c"], prev["v_c"], prev["tok_off"], cur_k,
                                cur_v, head_role, mask, budget_m, T, Fc, query_stride, scale)
        r["ids"] = [[prev_ids[h][f] for f in r["kept"][h]] + list(range(first, first + Fc))
                    for h in range(H)]
        r["mask"] = mask
        out.append(r)
    return out


def profile_masses(q, k, tokens_per_frame: int, query_stride: int = 1,
                   scale: float = 0.0) -> np.ndarray:
    """Offline head profiling ([S] 关键模块 › 1): the attention mass every
    head puts on every window frame, averaged over the current chunk's
    queries (rows 0, s, 2s, ...; s = 1 takes them all), softmax over the
    whole window.  Returns [H, F_total]; each row sums to 1."""
    q = as_f64(q)
    k = as_f64(k)
    H, D = q.shape[1], q.shape[2]
    sc = logit_scale(D, scale)
    return np.stack([frame_masses(q[:, h, :], k[:, h, :], tokens_per_frame, query_stride,
                                  sc).mean(axis=0) for h in range(H)])


def chunk_discontinuity(mass_row: np.ndarray, cur_frames: int) -> float:
    """Reading of the pages' chunk-discontinuity indicator at frame
    granularity ([S] 关键模块 › 1: static heads concentrate on the chunk's start
    and end positions): the mean mass of the boundary frames (sink, first and
    last frame of each aligned F_c-frame chunk; window frame f has id f) over
    the mean mass of the other frames.  NaN when every frame is a boundary
    (F_c <= 2) or the other frames get no mass."""
    b = np.array([is_chunk_boundary(f, cur_frames) for f in range(len(mass_row))])
    if b.all() or not (~b).any():
        return float("nan")
    inner = float(np.mean(mass_row[~b]))
    return float(np.mean(mass_row[b]) / inner) if inner > 0 else float("nan")


def classify_heads(mass_sum: np.ndarray, n_calls: int, hist_frames: int, cur_frames: int,
                   threshold: float):
    """Head labels from profiled masses (summed over n_calls calls): a head
    is static when its chunk discontinuity is at least `threshold` (NaN is
    not), else dynamic.  A static head's keep mask marks the history frames
    whose mean mass is at least the uniform share 1 / F_total ([S] 关键模块 › 2:
    the fixed positions that matter, frozen after profiling).
    Returns (head_role [H] uint8, static_keep_mask [H, F_h] uint8, disc [H])."""
    mass = np.asarray(mass_sum, dtype=np.float64) / n_calls
    H, F_tot = mass.shape
    role = np.full(H, DYNAMIC, dtype=np.uint8)
    mask = np.zeros((H, hist_frames), dtype=np.uint8)
    disc = np.array([chunk_discontinuity(mass[h], cur_frames) for h in range(H)])
    for h in range(H):
        if disc[h] >= threshold:
            role[h] = STATIC
            mask[h] = mass[h, :hist_frames] >= 1.0 / F_tot
    return role, mask, disc


# ---- token-granular variant -------------------------------------------------

def static_token_keep(hist_frames: int, tokens_per_frame: int, cur_frames: int,
                      sink_frames: int, boundary_tokens: int) -> np.ndarray:
    """Token-granular static pattern ([S] 关键模块 › 1 and 2: static heads attend
    to the start and end tokens of a chunk, and keep those positions): the
    tokens of the first sink_frames history frames, plus the first and the last
    boundary_tokens tokens of every aligned history chunk of F_c frames (a
    trailing partial chunk included).  Sorted history token indices."""
    T, Fh = tokens_per_frame, hist_frames
    n = Fh * T
    keep = np.zeros(n, dtype=bool)
    keep[:min(sink_frames, Fh) * T] = True
    L = boundary_tokens
    for start in range(0, Fh, cur_frames):
        lo, hi = start * T, min(start + cur_frames, Fh) * T
        keep[lo:min(lo + L, hi)] = True
        keep[max(hi - L, lo):hi] = True
    return np.flatnonzero(keep).astype(np.int64)


def participative_scores(q_h: np.ndarray, k_cand: np.ndarray, query_stride: int) -> np.ndarray:
    """Importance of each candidate token j of one head: the summed dot products
    with the sampled current-chunk queries, phi_j = sum_r q_r . k_j (the
    participative rule on the Deep Forcing page, 3.1 动态token筛选算法: each
    candidate scored by the attention logits the recent queries give it;
    here the recent queries are the strided sample of the current chunk).
    Written as the double sum, float64."""
    rows = sampled_query_rows(q_h.shape[0], query_stride)
    return (as_f64(q_h)[rows] @ as_f64(k_cand).T).sum(axis=0)


def select_top_tokens(phi: np.ndarray, budget: int) -> np.ndarray:
    """The min(C, n) candidates ranked first by (phi descending, index
    ascending), returned in ascending order (Top-C selection)."""
    n = len(phi)
    c = min(max(budget, 0), n)
    order = sorted(range(n), key=lambda j: (-phi[j], j))
    return np.array(sorted(order[:c]), dtype=np.int64)


def compress_tokens(q, k, v, head_role, tokens_per_frame: int, hist_frames: int,
                    cur_frames: int, query_stride: int, sink_frames: int, recent_frames: int,
                    budget_tokens: int, boundary_tokens: int) -> Dict[str, object]:
    """Token-granular compression of one layer (plain window).

    Static head: static_token_keep.  Dynamic head: the history is cut into a
    sink (first sink_frames frames, kept), a recent zone (last recent_frames
    frames, kept) and the candidates between them, of which the top
    budget_tokens by participative score are kept ([Deep Forcing page] 3.1:
    Sink / Recent / Candidate zones, Top-C with C the remaining budget).
    Compacted rows per head: kept history tokens ascending, then the current
    chunk.  Returns src (per head, the window token index of every compacted
    row), k_c, v_c, tok_off and phi (per dynamic head, candidate scores).
    """
    T, Fh, Fc = tokens_per_frame, hist_frames, cur_frames
    H = len(head_role)
    n_hist = Fh * T
    s_tok = min(sink_frames, Fh) * T
    r_tok = min(recent_frames, max(Fh - min(sink_frames, Fh), 0)) * T
    cand_lo, cand_hi = s_tok, n_hist - r_tok
    src, phi = [], {}
    for h in range(H):
        if head_role[h] == DYNAMIC:
            p = participative_scores(q[:, h], k[cand_lo:cand_hi, h], query_stride)
            phi[h] = p
            sel = select_top_tokens(p, budget_tokens) + cand_lo
            hist = np.concatenate([np.arange(0, s_tok), sel, np.arange(cand_hi, n_hist)])
        else:
            hist = static_token_keep(Fh, T, Fc, sink_frames, boundary_tokens)
        src.append(np.concatenate([hist, np.arange(n_hist, n_hist + Fc * T)]).astype(np.int64))
    tok_off = np.zeros(H + 1, dtype=np.int64)
    for h in range(H):
        tok_off[h + 1] = tok_off[h] + len(src[h])
    D = k.shape[2]
    k_c = np.empty((int(tok_off[H]), D), dtype=k.dtype)
    v_c = np.empty((int(tok_off[H]), D), dtype=v.dtype)
    for h in range(H):
        k_c[tok_off[h]:tok_off[h + 1]] = k[src[h], h]
        v_c[tok_off[h]:tok_off[h + 1]] = v[src[h], h]
    return dict(src=src, k_c=k_c, v_c=v_c, tok_off=tok_off, phi=phi,
                cand=(cand_lo, cand_hi))


# ---- FP8 (OCP e4m3) compressed cache ----------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 e4m3 codes -> exact float64: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; the
    finite maximum is 0x7E = 448 and 0x7F / 0xFF are NaN (the format's
    definition in the OCP 8-bit floating point specification)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return sign * v


def e4m3_encode(x32: np.ndarray) -> np.ndarray:
    """float32 values -> e4m3 codes, round to nearest with ties to even,
    magnitudes above 448 saturated to 448.  Written from the format: in
    binade E (value in [2^E, 2^(E+1)), E >= -6; below 2^-6 the subnormal
    step of the E = -6 binade applies) the representable values are
    r * 2^(E-3) with r integer, and their codes are (E + 6) * 8 + r, a
    monotone numbering in which r = 16 rolls over into the next binade."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, e = np.frexp(a)
    E = np.maximum(e - 1, -6)
    r = np.round(a / np.ldexp(1.0, E - 3))          # numpy rounds halves to even
    code = np.where(a == 0, 0, (E + 6) * 8 + r).astype(np.int64)
    code = np.minimum(code, 0x7E)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_e4m3(x, scale: float) -> np.ndarray:
    """Per-tensor scaled quantization: code of float32(x) / float32(scale)
    (an IEEE float32 division, then e4m3_encode).  x: float32 values or bf16
    bit patterns."""
    xf = decode_bf16(x).astype(np.float32) if np.asarray(x).dtype == np.uint16 \
        else np.asarray(x, dtype=np.float32)
    return e4m3_encode(xf / np.float32(scale))


def compress_fp8(q, k, v, head_role, static_keep_mask, budget_m: int, tokens_per_frame: int,
                 hist_frames: int, cur_frames: int, query_stride: int, k_scale, v_scale,
                 scale: float = 0.0) -> Dict[str, np.ndarray]:
    """compress() with the compacted rows stored as e4m3 codes: row j of head
    h holds quantize_e4m3(k_row, k_scale[h]) (and v likewise) -- the pages
    stack the method with quantization to compress memory further."""
    r = compress(q, k, v, head_role, static_keep_mask, budget_m, tokens_per_frame, hist_frames,
                 cur_frames, query_stride, scale)
    H = len(head_role)
    k8 = np.empty(r["k_c"].shape, dtype=np.uint8)
    v8 = np.empty(r["v_c"].shape, dtype=np.uint8)
    for h in range(H):
        lo, hi = int(r["tok_off"][h]), int(r["tok_off"][h + 1])
        k8[lo:hi] = quantize_e4m3(r["k_c"][lo:hi], k_scale[h])
        v8[lo:hi] = quantize_e4m3(r["v_c"][lo:hi], v_scale[h])
    r["k8"], r["v8"] = k8, v8
    return r


def attend_fp8(q, k8, v8, tok_off, q_scale, k_scale, v_scale, scale: float = 0.0,
               rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Attention with e4m3 operands: the queries are quantized per head
    (quantize_e4m3(q, q_scale[h])), keys and values are the cache's codes;
    everything is then decoded exactly and attention runs in float64 on
    q_hat * q_scale, k_hat * k_scale, v_hat * v_scale.  (Rounding the softmax
    weights for an fp8 value product is the kernel's own approximation and
    is not modelled here.)"""
    H = q.shape[1]
    qf = np.empty(q.shape, dtype=np.float64)
    for h in range(H):
        qf[:, h] = e4m3_decode(quantize_e4m3(q[:, h], q_scale[h])) * np.float64(q_scale[h])
    kf = np.empty(k8.shape, dtype=np.float64)
    vf = np.empty(v8.shape, dtype=np.float64)
    for h in range(H):
        lo, hi = int(tok_off[h]), int(tok_off[h + 1])
        kf[lo:hi] = e4m3_decode(k8[lo:hi]) * np.float64(k_scale[h])
        vf[lo:hi] = e4m3_decode(v8[lo:hi]) * np.float64(v_scale[h])
    return attend(qf, kf, vf, tok_off, scale, rows)


def cutoff_band(score_row: np.ndarray, budget_m: int, rel: float = TIE_REL):
    """Frames whose membership in the top-m set is decided by a near tie.

    When the m_eff-th and the (m_eff+1)-th best scores differ by at most
    ``rel`` relative, every frame whose score lies within ``rel`` (relative)
    of the m_eff-th best is ambiguous: another exact arithmetic order may keep
    any m_eff-sized set that holds all frames above the band and none below.
    Returns (sure_keep, band, sure_drop) as sets of frame indices.
    """
    f_h = len(score_row)
    m_eff = min(budget_m, f_h)
    order = sorted(range(f_h), key=lambda f: (-score_row[f], f))
    if m_eff == 0 or m_eff == f_h:
        return set(order[:m_eff]), set(), set(order[m_eff:])
    s_m, s_n = score_row[order[m_eff - 1]], score_row[order[m_eff]]
    if abs(s_m - s_n) > rel * max(abs(s_m), abs(s_n)):
        return set(order[:m_eff]), set(), set(order[m_eff:])
    band = {f for f in range(f_h)
            if abs(score_row[f] - s_m) <= rel * max(abs(score_row[f]), abs(s_m))}
    keep = {f for f in order[:m_eff] if f not in band}
    drop = {f for f in order[m_eff:] if f not in band}
    return keep, band, drop


def kept_set_valid(candidate: Sequence[int], score_row: np.ndarray, budget_m: int,
                   rel: float = TIE_REL) -> bool:
    """Whether a kept set agrees with the oracle up to the cutoff tie band."""
    keep, band, drop = cutoff_band(score_row, budget_m, rel)
    g = set(int(x) for x in candidate)
    m_eff = min(budget_m, len(score_row))
    return len(g) == m_eff and keep <= g and not (g & drop) and g <= (keep | band)
