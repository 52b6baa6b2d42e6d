"""Benchmark of the Forcing-KV hot path on one MI355X.

One step = one pass of the whole path over one attention layer:
fkv_compress_attend, i.e. fkv_compress (score dynamic heads, select frames,
compact K/V) then fkv_attend (the current chunk's queries over the
compressed cache) in one call, which starts the attention of the heads
without scored frames beside the scoring of the others when the attention
runs one workgroup per (head, query tile).  The same pass as the two calls
is reported as breakdown_ms.step_two_calls.  Inputs are seeded
synthetic tensors already resident in HBM.  The default workload is the
480P single layer (12 heads, D=128, 1560 tokens per latent frame, 18 history
+ 3 current frames, m=13, every 16th query scored); the 1080P layer is
measured too and reported under "secondary".

To keep the 256 MB last-level cache from holding a 480P layer's whole window
between steps, the timed loop walks over several device copies of the layer
(--copies), so K/V come from HBM as they would in a multi-layer pass.

The multi-layer passes (the 30-layer 480P pass and the 40-layer 720P pass of
a 14B-class model) are timed with every layer's inputs and compressed cache
resident in HBM at once ("multi_layer").

Also reported (same workload): the rolling compressed cache at its settled
size ("rolling"), head profiling over every query of a sample
("head_profiling"), the token-granular variant ("token_variant"), the e4m3
cache with fp8 attention ("fp8_cache", 480P and 1080P), and the CPU oracle
on the host ("cpu_baseline": the 480P layer in full, and under "configs" the
oracle's time on layer 0 of the other workloads, extrapolated where stated).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
HBM_PEAK_GBS = 8000.0
METRIC = "compressed-attn query tok/s per layer @480P/1080P; % MFMA & HBM roofline"
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--clock-warmup", type=float, default=0.5,
                    help="seconds of untimed steps before the first timed loop of a "
                         "workload (the GPU's clocks ramp up under load; without it the "
                         "first loop of a fresh process runs a few percent slow)")
    ap.add_argument("--workload", default="480p_layer")
    ap.add_argument("--secondary", default="1080p_layer",
                    help="second workload to report ('' to skip)")
    ap.add_argument("--copies", type=int, default=4,
                    help="device copies of layer 0 that the timed loops cycle over")
    ap.add_argument("--layers", type=int, default=0,
                    help="cycle over the workload's first N layers (own seeds, roles and "
                         "masks) instead of copies of layer 0")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-configs", default="tiny_f32,1080p_layer,480p_30layers,720p_14b_40layers",
                    help="further workloads whose oracle time is reported under "
                         "cpu_baseline.configs (layer 0; '' to skip)")
    ap.add_argument("--no-rolling", action="store_true",
                    help="skip the rolling-cache measurement")
    ap.add_argument("--multilayer", default="480p_30layers,720p_14b_40layers",
                    help="multi-layer passes to time with every layer resident "
                         "(comma-separated workload names, '' to skip)")
    ap.add_argument("--profile-only", action="store_true",
                    help="run the timed loop only (for rocprofv3), print nothing else")
    ap.add_argument("--only", choices=["step", "two_calls", "compress", "attend", "dense", "copy"],
                    default="step",
                    help="with --profile-only: which call the loop runs ('copy': a plain "
                         "1 GiB device-to-device tensor copy, the reference for counter "
                         "calibration)")
    return ap.parse_args()


class Layer:
    """Device state of one layer (inputs + compressed cache + outputs).  With
    `src`, the inputs are device copies of another Layer's."""

    def __init__(self, w, inp, fkv, torch, src=None):
        self.w = w
        if src is None:
            self.q, self.k, self.v = (fkv.to_device(inp.q), fkv.to_device(inp.k),
                                      fkv.to_device(inp.v))
        else:
            self.q, self.k, self.v = src.q.clone(), src.k.clone(), src.v.clone()
        self.role, self.mask = inp.head_role, inp.static_keep_mask
        self.desc = fkv.desc_for(w)
        self.ckv = fkv.CompressedKV(self.desc, self.role, self.mask, w.budget_m)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.out = torch.empty((w.n_q, w.num_heads, w.head_dim), dtype=dt, device="cuda")
        self.dout = torch.empty_like(self.out)


def note(msg):
    """One line on stderr as each stage of the run ends (stdout carries only
    the JSON result)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def clock_warmup(fn, layers, seconds, torch):
    """Untimed calls of fn for about `seconds` (synchronising every 16
    calls), so that the timed loops that follow run at the clocks of a
    loaded GPU."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        fn(layers[i % len(layers)])
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_loop(fn, layers, steps, warmup, torch):
    """Mean ms per call of fn(layer), cycling through layers; events on the
    stream the kernels are launched on (torch's current stream)."""
    for i in range(warmup):
        fn(layers[i % len(layers)])
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(layers[i % len(layers)])
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def measure(wname, args, fkv, torch, W):
    w = W.WORKLOADS[wname]
    inp = W.generate_layer(w, 0)
    base = Layer(w, inp, fkv, torch)
    if args.layers > 1:
        layers = [base] + [Layer(w, W.generate_layer(w, l), fkv, torch)
                           for l in range(1, min(args.layers, w.num_layers))]
    else:
        layers = [base] + [Layer(w, inp, fkv, torch, src=base)
                           for _ in range(max(args.copies, 1) - 1)]

    # One step = one layer's compression and attention, as one call
    # (fkv_compress_attend, the attention workspace of the layer's cache);
    # the same pass as the two calls fkv_compress + fkv_attend is timed too.
    def step(L):
        fkv.fkv_compress_attend(L.desc, L.q, L.k, L.v, L.role, L.mask, w.budget_m, L.ckv, L.out)

    def step_two_calls(L):
        fkv.fkv_compress(L.desc, L.q, L.k, L.v, L.role, L.mask, w.budget_m, L.ckv)
        fkv.fkv_attend(L.desc, L.q, L.ckv, L.out)

    if args.profile_only:
        fn = {"step": step, "two_calls": step_two_calls,
              "compress": lambda L: fkv.fkv_compress(L.desc, L.q, L.k, L.v, L.role, L.mask,
                                                     w.budget_m, L.ckv),
              "attend": lambda L: fkv.fkv_attend(L.desc, L.q, L.ckv, L.out),
              "dense": lambda L: fkv.fkv_attend_dense(L.desc, L.q, L.k, L.v, L.dout,
                                                     L.ckv.attend_ws)}[args.only]
        if args.only == "attend":
            for L in layers:
                step(L)
        time_loop(fn, layers, args.steps, args.warmup, torch)
        return None
    clock_warmup(step, layers, args.clock_warmup, torch)
    ms_step = time_loop(step, layers, args.steps, args.warmup, torch)
    ms_step_two_calls = time_loop(step_two_calls, layers, args.steps, args.warmup, torch)
    ms_compress = time_loop(lambda L: fkv.fkv_compress(L.desc, L.q, L.k, L.v, L.role, L.mask,
                                                       w.budget_m, L.ckv),
                            layers, args.steps, args.warmup, torch)
    ms_attend = time_loop(lambda L: fkv.fkv_attend(L.desc, L.q, L.ckv, L.out),
                          layers, args.steps, args.warmup, torch)
    ms_dense = time_loop(lambda L: fkv.fkv_attend_dense(L.desc, L.q, L.k, L.v, L.dout,
                                                         L.ckv.attend_ws),
                         layers, args.steps, args.warmup, torch)
    # per-stage times of the compression (HIP events around each kernel)
    stages = []
    for i in range(max(args.steps // 4, 5)):
        L = layers[i % len(layers)]
        stages.append(fkv.fkv_compress_timed(L.desc, L.q, L.k, L.v, L.role, L.mask,
                                             w.budget_m, L.ckv))
    stage_ms = [float(np.median([x[j] for x in stages])) for j in range(3)]
    kept = sum(L.ckv.kept_tokens for L in layers) / len(layers)  # mean over the layers
    D = w.head_dim
    attn_flop = 4.0 * w.n_q * D * kept
    dense_flop = 4.0 * w.n_q * D * w.n_win * w.num_heads
    elt = 2 if w.dtype == "bf16" else 4
    return dict(w=w, inp=inp, kept=kept, ms_step=ms_step, ms_step_two_calls=ms_step_two_calls,
                ms_compress=ms_compress,
                stage_ms=stage_ms,
                ms_attend=ms_attend, ms_dense=ms_dense, attn_flop=attn_flop,
                dense_flop=dense_flop, n_layers=len(layers),
                compact_bytes=4.0 * kept * D * elt,
                kept_frac_hist=(kept / w.num_heads / w.tokens_per_frame - w.cur_frames)
                / max(w.hist_frames, 1))


def measure_multilayer(wname, args, fkv, torch, W, reps):
    """A whole multi-layer pass with every layer resident in HBM: one chunk
    step of all layers (fkv_compress_attend per layer, in layer order),
    the same pass's attention alone, and the full-KV attention pass
    (fkv_attend_dense per layer).  Layers are generated on the host by a few
    threads (NumPy releases the interpreter lock in its array loops) and
    uploaded as they are ready."""
    import concurrent.futures as cf
    w = W.WORKLOADS[wname]
    layers = [None] * w.num_layers
    t0 = time.perf_counter()
    workers = max(1, min(8, len(os.sched_getaffinity(0)) // 2))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {ex.submit(W.generate_layer, w, l): l for l in range(w.num_layers)}
        for f in cf.as_completed(futs):
            l = futs[f]
            layers[l] = Layer(w, f.result(), fkv, torch)
            del futs[f]
    gen_s = time.perf_counter() - t0

    def run_pass(fn):
        for L in layers:
            fn(L)

    def step(L):
        fkv.fkv_compress_attend(L.desc, L.q, L.k, L.v, L.role, L.mask, w.budget_m, L.ckv, L.out)

    clock_warmup(lambda _: run_pass(step), [None], args.clock_warmup, torch)
    ms_pass = time_loop(lambda _: run_pass(step), [None], reps, 1, torch)
    ms_attend = time_loop(lambda _: run_pass(lambda L: fkv.fkv_attend(L.desc, L.q, L.ckv,
                                                                      L.out)),
                          [None], reps, 1, torch)
    ms_dense = time_loop(lambda _: run_pass(lambda L: fkv.fkv_attend_dense(
        L.desc, L.q, L.k, L.v, L.dout, L.ckv.attend_ws)), [None], reps, 1, torch)
    rows = sum(L.ckv.kept_tokens for L in layers)
    n = w.num_layers
    flop = 4.0 * w.n_q * w.head_dim * rows
    elt = 2 if w.dtype == "bf16" else 4
    resident = sum(t.numel() * t.element_size()
                   for L in layers for t in (L.q, L.k, L.v, L.ckv.k, L.ckv.v, L.out, L.dout))
    out = {"workload": w.name, "layers": n, "passes_timed": reps,
           "value": w.n_q * n / (ms_pass * 1e-3), "unit": "query tok/s per layer",
           "ms_per_pass": ms_pass, "ms_per_layer": ms_pass / n,
           "ms_attend_pass": ms_attend, "ms_full_kv_attend_pass": ms_dense,
           "attend_tflops": flop / (ms_attend * 1e-3) / 1e12,
           "attend_frac_of_peak": flop / (ms_attend * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
           "speedup_vs_full_kv": ms_dense / ms_pass,
           "attention_speedup_vs_full_kv": ms_dense / ms_attend,
           "kept_fraction_of_history_kv":
               (rows / n / w.num_heads / w.tokens_per_frame - w.cur_frames) / w.hist_frames,
           "cache_bytes_full": 2.0 * n * w.n_win * w.num_heads * w.head_dim * elt,
           "cache_bytes_compressed": 2.0 * rows * w.head_dim * elt,
           "hbm_resident_bytes": float(resident), "host_generation_s": gen_s}
    del layers
    torch.cuda.empty_cache()
    return out


def measure_rolling(wname, args, fkv, torch, W, n_chunks=8):
    """The cache carried across chunk steps (RollingCache): run n_chunks - 1
    chunks so that every head's history has settled, then time, on the last
    chunk's inputs, (a) a chunk step with fresh selection
    (fkv_compress_ragged + fkv_attend) and (b) a later denoising step of the
    same chunk with the selection reused (fkv_refresh_current + fkv_attend).
    Memory: the settled cache against the plain window's K/V."""
    w = W.WORKLOADS[wname]
    ro = W.generate_rollout(w, n_chunks)
    T, Fh, Fc, H = w.tokens_per_frame, w.hist_frames, w.cur_frames, w.num_heads
    desc = fkv.desc_for(w)
    rc = fkv.RollingCache(desc, ro.head_role, w.budget_m)
    k_all, v_all = fkv.to_device(ro.k), fkv.to_device(ro.v)
    qs = [fkv.to_device(q) for q in ro.q]
    sizes = []
    for c in range(n_chunks - 1):
        lo, hi = (Fh + c * Fc) * T, (Fh + (c + 1) * Fc) * T
        if c == 0:
            rc.step(qs[0], k_all[lo:hi], v_all[lo:hi], window_k=k_all[:hi], window_v=v_all[:hi])
        else:
            rc.step(qs[c], k_all[lo:hi], v_all[lo:hi])
        sizes.append(rc.rows)
    torch.cuda.synchronize()
    c = n_chunks - 1
    lo, hi = (Fh + c * Fc) * T, (Fh + (c + 1) * Fc) * T
    cur_k, cur_v, q = k_all[lo:hi], v_all[lo:hi], qs[c]
    hist = rc.cache
    hist_frames = [len(x) for x in rc.ids]
    mask = rc._masks(rc.ids)
    out_ckv = rc.bufs[rc.which ^ 1]
    out = torch.empty((w.n_q, H, w.head_dim), dtype=torch.bfloat16, device="cuda")

    def chunk_step(_):
        fkv.fkv_compress_ragged(desc, q, hist, hist_frames, cur_k, cur_v, ro.head_role, mask,
                                w.budget_m, out_ckv)
        fkv.fkv_attend(desc, q, out_ckv, out, hist.attend_ws)

    def reuse_step(_):
        fkv.fkv_refresh_current(desc, cur_k, cur_v, out_ckv)
        fkv.fkv_attend(desc, q, out_ckv, out, hist.attend_ws)

    clock_warmup(chunk_step, [None], args.clock_warmup, torch)
    ms_chunk = time_loop(chunk_step, [None], args.steps, args.warmup, torch)
    ms_reuse = time_loop(reuse_step, [None], args.steps, args.warmup, torch)
    rows, _ = fkv.fkv_plan_ragged(desc, hist_frames, ro.head_role, mask, w.budget_m)
    elt = 2 if w.dtype == "bf16" else 4
    kv_bytes = lambda r: 2.0 * r * w.head_dim * elt
    return {
        "workload": w.name, "chunks_run": n_chunks,
        "cache_rows_per_chunk": sizes + [rows],
        "history_frames_per_head": hist_frames,
        "ms_chunk_step_reselect": ms_chunk, "ms_step_selection_reused": ms_reuse,
        "value_reselect": w.n_q / (ms_chunk * 1e-3),
        "value_selection_reused": w.n_q / (ms_reuse * 1e-3),
        "cache_bytes_settled": kv_bytes(rows),
        "window_bytes_plain": kv_bytes(w.n_win * H),
        "cache_reduction_vs_plain_window": 1.0 - rows / float(w.n_win * H),
    }


def measure_tokens(wname, args, fkv, torch, W):
    """Token-granular variant on one layer: sink frame, the last chunk as the
    recent zone, nine frames' worth of candidate tokens per dynamic head, half
    a frame at each chunk end for static heads.  Times fkv_compress_tokens
    and a step (compress + attend)."""
    w = W.WORKLOADS[wname]
    T = w.tokens_per_frame
    inp = W.generate_layer(w, 0)
    L = Layer(w, inp, fkv, torch)
    cfg = fkv.FkvTokenCfg(1, w.cur_frames, 9 * T, T // 2)
    ckv = fkv.CompressedKV(L.desc, inp.head_role, None, 0, token_cfg=cfg)

    def compress(_):
        fkv.fkv_compress_tokens(L.desc, cfg, L.q, L.k, L.v, inp.head_role, ckv)

    def step(_):
        compress(None)
        fkv.fkv_attend(L.desc, L.q, ckv, L.out)

    clock_warmup(step, [None], args.clock_warmup, torch)
    ms_c = time_loop(compress, [None], args.steps, args.warmup, torch)
    ms_s = time_loop(step, [None], args.steps, args.warmup, torch)
    return {"workload": w.name,
            "config": {"sink_frames": 1, "recent_frames": w.cur_frames,
                       "budget_tokens": 9 * T, "boundary_tokens": T // 2},
            "kept_rows": ckv.kept_tokens,
            "kept_fraction_of_window": ckv.kept_tokens / float(w.n_win * w.num_heads),
            "ms_compress": ms_c, "ms_per_step": ms_s, "value": w.n_q / (ms_s * 1e-3)}


def measure_fp8(wname, args, fkv, torch, W):
    """The e4m3 compressed cache on one layer: fkv_compress_fp8 +
    fkv_attend_fp8 per step (per-head scales amax / 448 of q, k, v), the
    attention's rate against the dense fp8 MFMA peak, cache bytes."""
    w = W.WORKLOADS[wname]
    inp = W.generate_layer(w, 0)
    L = Layer(w, inp, fkv, torch)
    H, D = w.num_heads, w.head_dim

    def scales(a):
        x = np.abs(W.bf16_bits_to_f32(a)).reshape(-1, H, D).max(axis=(0, 2))
        return np.maximum(x, 1e-6).astype(np.float32) / np.float32(448.0)

    ks, vs, qs = scales(inp.k), scales(inp.v), scales(inp.q)
    ckv = fkv.CompressedKV(L.desc, inp.head_role, inp.static_keep_mask, w.budget_m, fp8=True)

    def compress(_):
        fkv.fkv_compress_fp8(L.desc, L.q, L.k, L.v, L.role, L.mask, w.budget_m, ks, vs, ckv)

    def attend(_):
        fkv.fkv_attend_fp8(L.desc, L.q, ckv, qs, ks, vs, L.out)

    def step(_):
        compress(None)
        attend(None)

    steps = args.steps if w.tokens_per_frame < 5000 else max(args.steps // 4, 3)
    clock_warmup(step, [None], args.clock_warmup, torch)
    ms_s = time_loop(step, [None], steps, args.warmup, torch)
    ms_c = time_loop(compress, [None], steps, args.warmup, torch)
    ms_a = time_loop(attend, [None], steps, args.warmup, torch)
    flop = 4.0 * w.n_q * D * ckv.kept_tokens
    tf = flop / (ms_a * 1e-3) / 1e12
    return {"workload": w.name, "ms_per_step": ms_s, "value": w.n_q / (ms_s * 1e-3),
            "ms_compress": ms_c, "ms_attend": ms_a, "attend_tflops": tf,
            "attend_frac_of_fp8_peak": tf / FP8_PEAK_TFLOPS,
            "cache_bytes": 2.0 * ckv.kept_tokens * D,
            "cache_bytes_bf16": 4.0 * ckv.kept_tokens * D}


def measure_profile(wname, args, fkv, torch, W, stride=1):
    """Head profiling over every query of one warm-up sample
    (fkv_profile_heads, query stride 1): time per call and the score
    product's rate, 2 Nq D N_win H FLOP."""
    w = W.WORKLOADS[wname]
    inp = W.generate_profile_sample(w, 0)
    desc = fkv.make_desc(w.num_heads, w.head_dim, w.tokens_per_frame, w.hist_frames,
                         w.cur_frames, stride, w.dtype)
    q, k = fkv.to_device(inp.q), fkv.to_device(inp.k)
    ws = torch.empty(fkv.fkv_profile_workspace(desc), dtype=torch.uint8, device="cuda")
    acc = torch.zeros((w.num_heads, w.frames), dtype=torch.float32, device="cuda")
    ms = time_loop(lambda _: fkv.fkv_profile_heads(desc, q, k, acc, ws), [None],
                   max(args.steps // 4, 3), 2, torch)
    n_s = -(-w.n_q // stride)
    flop = 2.0 * n_s * w.head_dim * w.n_win * w.num_heads
    return {"workload": w.name, "query_stride": stride, "ms_per_sample": ms,
            "score_tflops": flop / (ms * 1e-3) / 1e12}


def kernel_rates(r):
    """Per-kernel times and rates of one measured workload: K1 scoring
    (2 n_s D N_win H_dyn FLOP against the bf16 peak), K2 selection (latency),
    K3 compaction (algorithmic bytes against HBM), K4 attention."""
    w = r["w"]
    s_ms, sel_ms, c_ms = r["stage_ms"]
    n_dyn = int((r["inp"].head_role == 1).sum())
    n_s = -(-w.n_q // w.query_stride)
    k1 = 2.0 * n_s * w.head_dim * w.n_win * n_dyn
    k1_tf = k1 / (s_ms * 1e-3) / 1e12 if s_ms > 0 else None
    k3_gbs = r["compact_bytes"] / (c_ms * 1e-3) / 1e9
    k4_tf = r["attn_flop"] / (r["ms_attend"] * 1e-3) / 1e12
    return {"score_us": s_ms * 1e3, "score_tflops": k1_tf,
            "score_frac_of_peak": k1_tf / BF16_PEAK_TFLOPS if k1_tf else None,
            "select_us": sel_ms * 1e3,
            "compact_us": c_ms * 1e3, "compact_gbs": k3_gbs,
            "compact_frac_of_hbm": k3_gbs / HBM_PEAK_GBS,
            "attend_us": r["ms_attend"] * 1e3, "attend_tflops": k4_tf,
            "attend_frac_of_peak": k4_tf / BF16_PEAK_TFLOPS}


def measured_peaks(fkv, torch):
    """The roofline denominators measured on this device: the sustained bf16
    MFMA rate (fkv_mfma_peak: chained 32x32x16 MFMAs on register operands)
    and a device-to-device copy of 1 GiB (bytes read + written / time)."""
    tf = fkv.fkv_mfma_peak()
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = time_loop(lambda _: dst.copy_(src), [None], 10, 2, torch)
    del src, dst
    return {"mfma_bf16_tflops": tf, "hbm_copy_gbs": 2.0 * (1 << 30) / (ms * 1e-3) / 1e9,
            "datasheet_bf16_tflops": BF16_PEAK_TFLOPS, "datasheet_hbm_gbs": HBM_PEAK_GBS}


def host_cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" elsewhere)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def numpy_blas() -> str:
    """Name and version of the BLAS NumPy was built against."""
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '?')}"
    except Exception:
        return "unknown"


def cpu_baseline(w, inp, min_seconds=10.0, max_reps=4):
    """The oracle as it stands, timed on this host over the whole layer
    (scoring, selection, compaction and attention of every query row),
    repeated until about min_seconds of work have run (at most max_reps)."""
    from oracle import forcing_kv as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    t_comp = t_attn = 0.0
    reps = 0
    while reps < max_reps and (t_comp + t_attn) < min_seconds:
        t0 = time.perf_counter()
        c = O.compress(inp.q, inp.k, inp.v, inp.head_role, inp.static_keep_mask, w.budget_m,
                       w.tokens_per_frame, w.hist_frames, w.cur_frames, w.query_stride)
        t1 = time.perf_counter()
        O.attend(inp.q, c["k_c"], c["v_c"], c["tok_off"])
        t2 = time.perf_counter()
        t_comp += t1 - t0
        t_attn += t2 - t1
        reps += 1
    return {"value": reps * w.n_q / (t_comp + t_attn), "unit": "query tok/s per layer",
            "cores": int(cores), "kind": "oracle",
            "cpu_model": host_cpu_model(), "blas": numpy_blas(),
            "sample": f"{w.name}: {reps} full layer pass(es), all {w.n_q} query rows: "
                      f"compress (score+select+compact) {t_comp:.1f} s + attention "
                      f"{t_attn:.1f} s; float64 NumPy"}



def cpu_baseline_config(name, W, rows=(64, 256), seed=11):
    """The oracle as it stands on layer 0 of another configuration: the
    compression (scoring, selection, compaction) timed in full, the attention
    of two seeded samples of query rows fitted as a + b * rows (the per-head
    conversion of the compressed rows is the fixed part a) and taken at every
    row.  Small workloads are timed in full.  A multi-layer pass is its
    layer count times layer 0 ("extrapolated")."""
    from oracle import forcing_kv as O
    w = W.WORKLOADS[name]
    inp = W.generate_layer(w, 0)
    t0 = time.perf_counter()
    c = O.compress(inp.q, inp.k, inp.v, inp.head_role, inp.static_keep_mask, w.budget_m,
                   w.tokens_per_frame, w.hist_frames, w.cur_frames, w.query_stride)
    t_comp = time.perf_counter() - t0
    if w.n_q <= 4 * rows[-1]:
        t0 = time.perf_counter()
        O.attend(inp.q, c["k_c"], c["v_c"], c["tok_off"])
        t_attn = time.perf_counter() - t0
        how = f"attention of all {w.n_q} query rows {t_attn:.2f} s"
    else:
        rng = np.random.default_rng(seed)
        t = []
        for n in rows:
            sel = rng.choice(w.n_q, n, replace=False)
            t0 = time.perf_counter()
            O.attend(inp.q, c["k_c"], c["v_c"], c["tok_off"], rows=sel)
            t.append(time.perf_counter() - t0)
        b = max((t[1] - t[0]) / (rows[1] - rows[0]), 0.0)
        a = max(t[0] - b * rows[0], 0.0)
        t_attn = a + b * w.n_q
        how = (f"attention of {rows[0]} and {rows[1]} sampled query rows ({t[0]:.2f} s, "
               f"{t[1]:.2f} s) fitted as a + b*rows and taken at all {w.n_q} rows "
               f"({t_attn:.1f} s)")
    t_layer = t_comp + t_attn
    out = {"workload": name, "value": w.n_q / t_layer, "unit": "query tok/s per layer",
           "s_per_layer": t_layer,
           "sample": f"layer 0: compress (score+select+compact) {t_comp:.1f} s in full; {how}",
           "extrapolated": w.n_q > 4 * rows[-1] or w.num_layers > 1}
    if w.num_layers > 1:
        out["s_per_pass"] = t_layer * w.num_layers
        out["sample"] += f"; pass = {w.num_layers} x layer 0"
    del inp, c
    return out

def traffic_record(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on this workload and on the current kernel source."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        import hashlib
        rec = json.load(open(path)).get(kernel)
        if rec["workload"] != workload:
            return None
        csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hybrid_kv_cache_amd",
                            "csrc")
        h = hashlib.sha256()
        for name in rec["sources"]:
            h.update(open(os.path.join(csrc, name), "rb").read())
        return rec["bytes_per_launch"] if h.hexdigest() == rec["sha256"] else None
    except Exception:
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the path needs no inter-GPU exchange; "
              f"--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from hybrid_kv_cache_amd import fkv
    from hybrid_kv_cache_amd import workloads as W
    fkv.load()

    if args.profile_only and args.only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        return
    r = measure(args.workload, args, fkv, torch, W)
    if args.profile_only:
        return
    note(f"{args.workload}: step {r['ms_step']:.4f} ms")
    w = r["w"]
    value = w.n_q / (r["ms_step"] * 1e-3)
    attn_tflops = r["attn_flop"] / (r["ms_attend"] * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "query tok/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "clock_warmup_s": args.clock_warmup,
        "ms_per_step": r["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded drift-plus-Gaussian q/k/v, no model weights)",
        "config": {"workload": w.name, "heads": w.num_heads, "head_dim": w.head_dim,
                   "tokens_per_frame": w.tokens_per_frame, "hist_frames": w.hist_frames,
                   "cur_frames": w.cur_frames, "query_tokens": w.n_q, "budget_m": w.budget_m,
                   "query_stride": w.query_stride,
                   **({"layers": r["n_layers"]} if args.layers > 1
                      else {"layer_copies": r["n_layers"]})},
        "roofline": {"bound": "mfma" if w.dtype == "bf16" else "alu",
                     "kernel": f"attend_{w.dtype} (fkv_attend)",
                     "achieved": attn_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": attn_tflops / peak, "traffic": traffic_record("attend", w.name)},
        "breakdown_ms": {"compress": r["ms_compress"], "attend": r["ms_attend"],
                         "attend_dense": r["ms_dense"],
                         "step_two_calls": r["ms_step_two_calls"]},
        "speedup_vs_full_kv": r["ms_dense"] / r["ms_step"],
        "attention_speedup_vs_full_kv": r["ms_dense"] / r["ms_attend"],
        "kept_fraction_of_history_kv": r["kept_frac_hist"],
        "compact_bytes_per_layer": r["compact_bytes"],
        "kernels": kernel_rates(r) if w.dtype == "bf16" else None,
    }
    if args.secondary:
        r2 = measure(args.secondary, args, fkv, torch, W)
        w2 = r2["w"]
        line["secondary"] = {
            "workload": w2.name, "value": w2.n_q / (r2["ms_step"] * 1e-3),
            "unit": "query tok/s per layer", "ms_per_step": r2["ms_step"],
            "breakdown_ms": {"compress": r2["ms_compress"], "attend": r2["ms_attend"],
                             "attend_dense": r2["ms_dense"],
                             "step_two_calls": r2["ms_step_two_calls"]},
            "attend_tflops": r2["attn_flop"] / (r2["ms_attend"] * 1e-3) / 1e12,
            "attend_frac_of_peak": r2["attn_flop"] / (r2["ms_attend"] * 1e-3) / 1e12 / peak,
            "speedup_vs_full_kv": r2["ms_dense"] / r2["ms_step"],
            "attention_speedup_vs_full_kv": r2["ms_dense"] / r2["ms_attend"],
            "kernels": kernel_rates(r2) if w2.dtype == "bf16" else None,
        }
        del r2
        note(f"{args.secondary}: step {line['secondary']['ms_per_step']:.4f} ms")
    if w.dtype == "bf16" and not args.no_rolling and args.layers <= 1:
        line["rolling"] = measure_rolling(w.name, args, fkv, torch, W)
        line["head_profiling"] = measure_profile(w.name, args, fkv, torch, W)
        line["token_variant"] = measure_tokens(w.name, args, fkv, torch, W)
        line["fp8_cache"] = [measure_fp8(n, args, fkv, torch, W)
                             for n in (w.name, args.secondary) if n]
        note("rolling cache, head profiling, token variant, e4m3 cache done")
    if w.dtype == "bf16" and args.multilayer and args.layers <= 1:
        line["multi_layer"] = [measure_multilayer(n, args, fkv, torch, W,
                                                  reps=5 if W.WORKLOADS[n].num_layers <= 30 else 3)
                               for n in args.multilayer.split(",") if n]
        note("multi-layer passes done")
    if w.dtype == "bf16":
        line["measured_peaks"] = measured_peaks(fkv, torch)
        line["roofline_frac_of_measured_peak"] = (
            line["roofline"]["achieved"] / line["measured_peaks"]["mfma_bf16_tflops"])
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, r["inp"])
        note(f"oracle on {w.name} done")
        line["cpu_baseline"]["configs"] = []
        for n in args.cpu_configs.split(","):
            if n:
                line["cpu_baseline"]["configs"].append(cpu_baseline_config(n, W))
                note(f"oracle on layer 0 of {n} done")
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
