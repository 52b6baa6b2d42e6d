"""Seeded synthetic workloads for the Forcing-KV hybrid compression path.

This module only builds inputs: shapes, head roles, static keep masks and
the drift-plus-Gaussian activations.  It contains none of the method's
arithmetic (no scoring, selection, compaction or attention), so both the CPU
oracle's tests and the GPU path may use it.

Shapes follow the chunk-wise autoregressive video DiT setting the Forcing-KV
pages describe (per-frame KV cache of a chunk-wise AR model, page
"Forcing-KV：面向高效自回归视频扩散模型的混合KV缓存压缩", section
方法 › 输入与整体流程): a window of ``hist_frames`` history latent frames
followed by the ``cur_frames`` frames of the current chunk, ``tokens_per_frame``
tokens per latent frame, all heads of one attention layer.

Tensor layout (token-major, as a fused QKV projection emits it):
  q        [Nq,    H, D]   Nq    = cur_frames * T
  k, v     [N_win, H, D]   N_win = (hist_frames + cur_frames) * T
Tokens are frame-major, oldest frame first; the current chunk is last.

The real activations of the pages' models (LongLive / Self Forcing on
Wan2.1-class backbones) are not available; these seeded tensors stand in for
them with the same shapes.
"""
from __future__ import annotations

import dataclasses
from typing import Iterator, List, Optional

import numpy as np

STATIC = 0
DYNAMIC = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "bf16" or "f32": storage type of q/k/v
    num_heads: int
    head_dim: int
    tokens_per_frame: int
    hist_frames: int
    cur_frames: int
    query_stride: int
    budget_m: int
    num_static: int            # heads labelled static per layer
    num_layers: int
    seed_base: int             # layer l uses seed_base + l (single layer: seed_base)
    fixed_static_heads: Optional[tuple] = None  # tiny case: roles fixed, not drawn
    description: str = ""

    @property
    def frames(self) -> int:
        return self.hist_frames + self.cur_frames

    @property
    def n_win(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def n_q(self) -> int:
        return self.cur_frames * self.tokens_per_frame

    @property
    def n_sampled(self) -> int:
        return -(-self.n_q // self.query_stride)

    def seed(self, layer: int = 0) -> int:
        return self.seed_base + layer


def latent_tokens(width: int, height: int, vae: int = 8, patch: int = 2) -> int:
    """Tokens per latent frame of a video DiT: (W/vae/patch) * (H/vae/patch)."""
    return (width // vae // patch) * (height // vae // patch)


# The five workloads.  480P = 832x480 -> 52*30 = 1560 tokens per latent frame;
# 720P = 1280x720 -> 80*45 = 3600; 1080P = 1920x1088 -> 120*68 = 8160.
WORKLOADS = {
    "tiny_f32": Workload(
        name="tiny_f32", dtype="f32", num_heads=4, head_dim=64, tokens_per_frame=64,
        hist_frames=6, cur_frames=3, query_stride=4, budget_m=4, num_static=2,
        num_layers=1, seed_base=0, fixed_static_heads=(0, 1),
        description="tiny fp32 single layer: 4 heads (0-1 static), D=64, T=64, "
                    "6 history + 3 current frames, m=4, every 4th query"),
    "480p_layer": Workload(
        name="480p_layer", dtype="bf16", num_heads=12, head_dim=128,
        tokens_per_frame=latent_tokens(832, 480), hist_frames=18, cur_frames=3,
        query_stride=16, budget_m=13, num_static=6, num_layers=1, seed_base=1,
        description="Wan2.1-1.3B-like layer at 480P: 12 heads (6 static), D=128, "
                    "T=1560, 18 history + 3 current frames, m=13, every 16th query"),
    "480p_30layers": Workload(
        name="480p_30layers", dtype="bf16", num_heads=12, head_dim=128,
        tokens_per_frame=latent_tokens(832, 480), hist_frames=18, cur_frames=3,
        query_stride=16, budget_m=13, num_static=5, num_layers=30, seed_base=2000,
        description="30-layer pass at 480P: per-layer seeds, 5 static / 7 dynamic "
                    "heads per layer (40/60), m=13 (about 70% of history KV kept)"),
    "1080p_layer": Workload(
        name="1080p_layer", dtype="bf16", num_heads=12, head_dim=128,
        tokens_per_frame=latent_tokens(1920, 1088), hist_frames=18, cur_frames=3,
        query_stride=32, budget_m=12, num_static=6, num_layers=1, seed_base=3,
        description="1080P layer: 12 heads (6 static), D=128, T=8160, 18 history + "
                    "3 current frames, m=12, every 32nd query"),
    "720p_14b_40layers": Workload(
        name="720p_14b_40layers", dtype="bf16", num_heads=40, head_dim=128,
        tokens_per_frame=latent_tokens(1280, 720), hist_frames=18, cur_frames=3,
        query_stride=16, budget_m=12, num_static=16, num_layers=40, seed_base=4000,
        description="Wan2.1-14B-like 40-layer pass at 720P: 40 heads (16 static), "
                    "D=128, T=3600, 18 history + 3 current frames, m=12, every 16th query"),
}


def chunk_boundary_mask(hist_frames: int, chunk: int = 3) -> np.ndarray:
    """Frame-level static keep pattern: the sink frame 0 plus the first and the
    last frame of every past chunk of ``chunk`` frames (a partial trailing
    chunk keeps its first and last existing frame)."""
    keep = np.zeros(hist_frames, dtype=np.uint8)
    if hist_frames == 0:
        return keep
    keep[0] = 1
    for start in range(0, hist_frames, chunk):
        keep[start] = 1
        keep[min(start + chunk, hist_frames) - 1] = 1
    return keep


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even.  Inputs are
    finite (the generator draws no NaN/Inf)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class LayerInputs:
    """One layer's inputs.  q/k/v hold float32 values for "f32" workloads and
    bf16 bit patterns (uint16) for "bf16" workloads; either way they are the
    exact values both sides consume."""
    workload: Workload
    layer: int
    q: np.ndarray              # [Nq, H, D]
    k: np.ndarray              # [N_win, H, D]
    v: np.ndarray              # [N_win, H, D]
    head_role: np.ndarray      # [H] uint8, 0 static / 1 dynamic
    static_keep_mask: np.ndarray  # [H, F_h] uint8 (rows of dynamic heads unused)
    target_frame: np.ndarray   # [H] history frame each head's queries lean to

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def generate_layer(w: Workload, layer: int = 0, *, zero_q: bool = False) -> LayerInputs:
    """Drift-plus-Gaussian generator.

    Draw order from Generator(PCG64(seed)):
      1. head roles: a permutation of the heads, the first ``num_static`` static
         (skipped when the roles are fixed);
      2. target frame per head, uniform over the history frames;
      3. drift mu[h, f, :], a random walk over the window's frames with
         N(0, 0.3^2) steps;
      4. keys: mu[h, frame(token)] + N(0, 1);
      5. values: N(0, 1);
      6. queries: N(0, 1) + 0.5 * mu[h, target[h]].
    All draws are float32 in [H, N, D] order, then moved to token-major
    [N, H, D].  bf16 workloads are then rounded to bf16 (RNE).
    """
    H, D, T = w.num_heads, w.head_dim, w.tokens_per_frame
    Fh, Ft = w.hist_frames, w.frames
    rng = np.random.Generator(np.random.PCG64(w.seed(layer)))

    role = np.full(H, DYNAMIC, dtype=np.uint8)
    if w.fixed_static_heads is not None:
        role[list(w.fixed_static_heads)] = STATIC
    else:
        role[rng.permutation(H)[: w.num_static]] = STATIC
    tgt = rng.integers(0, max(Fh, 1), H)

    mu = np.cumsum(np.float32(0.3) * rng.standard_normal((H, Ft, D), dtype=np.float32),
                   axis=1, dtype=np.float32)
    k = rng.standard_normal((H, Ft, T, D), dtype=np.float32)
    k += mu[:, :, None, :]
    v = rng.standard_normal((H, w.n_win, D), dtype=np.float32)
    q = rng.standard_normal((H, w.n_q, D), dtype=np.float32)
    q += np.float32(0.5) * mu[np.arange(H), tgt][:, None, :]
    if zero_q:
        q[...] = 0.0

    k = k.reshape(H, w.n_win, D)

    def to_token_major(a):
        t = np.ascontiguousarray(a.transpose(1, 0, 2))
        return round_to_bf16_bits(t) if w.dtype == "bf16" else t

    mask = np.tile(chunk_boundary_mask(Fh, w.cur_frames), (H, 1))
    out = LayerInputs(workload=w, layer=layer, q=to_token_major(q),
                      k=to_token_major(k), v=to_token_major(v), head_role=role,
                      static_keep_mask=np.ascontiguousarray(mask, dtype=np.uint8),
                      target_frame=tgt)
    return out


@dataclasses.dataclass
class RolloutInputs:
    """Inputs of n_chunks consecutive chunk steps of one layer.  Frame store
    k / v [(F_h + n_chunks F_c) T, H, D] token-major: chunk 0's window is
    frames [0, F_h + F_c), chunk c's current frames are
    [F_h + c F_c, F_h + (c + 1) F_c).  q[c] [Nq, H, D] are chunk c's queries.
    Same value conventions as LayerInputs."""
    workload: Workload
    n_chunks: int
    q: List[np.ndarray]
    k: np.ndarray
    v: np.ndarray
    head_role: np.ndarray
    static_keep_mask: np.ndarray   # [H, F_h]: chunk 0's window (frame ids 0 .. F_h - 1)

    def window(self) -> LayerInputs:
        """Chunk 0 as a plain one-layer window."""
        w = self.workload
        n = w.n_win
        return LayerInputs(workload=w, layer=0, q=self.q[0], k=self.k[:n], v=self.v[:n],
                           head_role=self.head_role, static_keep_mask=self.static_keep_mask,
                           target_frame=np.zeros(w.num_heads, dtype=np.int64))

    def current(self, name: str, c: int) -> np.ndarray:
        """Chunk c's current-frame rows of k or v: [F_c T, H, D]."""
        w = self.workload
        lo = (w.hist_frames + c * w.cur_frames) * w.tokens_per_frame
        return getattr(self, name)[lo:lo + w.cur_frames * w.tokens_per_frame]


def generate_rollout(w: Workload, n_chunks: int, seed: Optional[int] = None) -> RolloutInputs:
    """Drift-plus-Gaussian generator over a longer frame sequence.

    Draw order from Generator(PCG64(seed or the workload's layer-0 seed)):
      1. head roles as in generate_layer;
      2. target frame per (chunk, head): uniform over the frames before that
         chunk's current frames;
      3. drift over all F_h + n_chunks F_c frames (N(0, 0.3^2) steps);
      4. keys mu + N(0, 1); 5. values N(0, 1);
      6. queries of each chunk: N(0, 1) + 0.5 mu[h, target[c, h]].
    """
    H, D, T = w.num_heads, w.head_dim, w.tokens_per_frame
    Fh, Fc = w.hist_frames, w.cur_frames
    F_all = Fh + n_chunks * Fc
    rng = np.random.Generator(np.random.PCG64(w.seed(0) if seed is None else seed))
    role = np.full(H, DYNAMIC, dtype=np.uint8)
    if w.fixed_static_heads is not None:
        role[list(w.fixed_static_heads)] = STATIC
    else:
        role[rng.permutation(H)[: w.num_static]] = STATIC
    tgt = np.stack([rng.integers(0, max(Fh + c * Fc, 1), H) for c in range(n_chunks)])
    mu = np.cumsum(np.float32(0.3) * rng.standard_normal((H, F_all, D), dtype=np.float32),
                   axis=1, dtype=np.float32)
    k = rng.standard_normal((H, F_all, T, D), dtype=np.float32)
    k += mu[:, :, None, :]
    v = rng.standard_normal((H, F_all * T, D), dtype=np.float32)
    qs = []
    for c in range(n_chunks):
        q = rng.standard_normal((H, w.n_q, D), dtype=np.float32)
        q += np.float32(0.5) * mu[np.arange(H), tgt[c]][:, None, :]
        qs.append(q)
    k = k.reshape(H, F_all * T, D)

    def to_token_major(a):
        t = np.ascontiguousarray(a.transpose(1, 0, 2))
        return round_to_bf16_bits(t) if w.dtype == "bf16" else t

    mask = np.tile(chunk_boundary_mask(Fh, Fc), (H, 1))
    return RolloutInputs(workload=w, n_chunks=n_chunks, q=[to_token_major(q) for q in qs],
                         k=to_token_major(k), v=to_token_major(v), head_role=role,
                         static_keep_mask=np.ascontiguousarray(mask, dtype=np.uint8))


def generate_profile_sample(w: Workload, sample: int = 0, strength: float = 4.0) -> LayerInputs:
    """A warm-up sample for head profiling: generate_layer's recipe with the
    seed of layer `sample` for the content, the head roles of layer 0 (roles
    belong to the model, not to the sample), plus a positional signature on
    the static heads: a unit direction u_h (one per head, from its own
    seeded generator) is added, times `strength`, to every query of the head
    and to the keys of its boundary frames (the sink and the first and last
    frame of every aligned chunk of F_c frames, current chunk included), so
    that these heads attend to chunk starts and ends as the pages describe
    static heads doing.  Dynamic heads are left as generate_layer makes them."""
    base = generate_layer(w, sample)
    base.head_role = generate_layer(small_copy(w), 0).head_role
    H, D, T, F = w.num_heads, w.head_dim, w.tokens_per_frame, w.frames
    rng = np.random.Generator(np.random.PCG64(w.seed(sample) + 7919))
    u = rng.standard_normal((H, D)).astype(np.float32)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    q = base.as_f32("q").copy()
    k = base.as_f32("k").copy()
    Fc = w.cur_frames
    boundary = [f for f in range(F) if f == 0 or f % Fc in (0, Fc - 1)]
    for h in range(H):
        if base.head_role[h] != STATIC:
            continue
        q[:, h] += np.float32(strength) * u[h]
        for f in boundary:
            k[f * T:(f + 1) * T, h] += np.float32(strength) * u[h]
    conv = (lambda a: round_to_bf16_bits(a)) if w.dtype == "bf16" else (lambda a: a)
    base.q, base.k = conv(np.ascontiguousarray(q)), conv(np.ascontiguousarray(k))
    return base


def small_copy(w: Workload) -> Workload:
    """The same workload with one-token frames (same seeds and head roles):
    cheap to generate when only the role draw is wanted."""
    return dataclasses.replace(w, tokens_per_frame=1, dtype="f32")


def iter_layers(w: Workload, layers: Optional[List[int]] = None) -> Iterator[LayerInputs]:
    for l in (range(w.num_layers) if layers is None else layers):
        yield generate_layer(w, l)


def small_workload(name: str = "small_bf16", *, dtype: str = "bf16", num_heads: int = 3,
                   head_dim: int = 128, tokens_per_frame: int = 100, hist_frames: int = 6,
                   cur_frames: int = 3, query_stride: int = 4, budget_m: int = 4,
                   num_static: int = 1, seed: int = 7) -> Workload:
    """A reduced-size workload for parity tests: same recipe, shapes the CPU
    oracle finishes in seconds, with ragged tails against 64-row tiles."""
    return Workload(name=name, dtype=dtype, num_heads=num_heads, head_dim=head_dim,
                    tokens_per_frame=tokens_per_frame, hist_frames=hist_frames,
                    cur_frames=cur_frames, query_stride=query_stride, budget_m=budget_m,
                    num_static=num_static, num_layers=1, seed_base=seed)
