// C ABI of libfkv.so (declared in include/fkv.h): argument checks, the
// data-independent plan (kept counts, offsets, workspace layout) and the
// launch sequence of the compression and attention kernels.
//
// The plan follows the method's split of heads (Forcing-KV, tomesphere page,
// Abstract; ai-feeds summary, 方法 › 关键模块 2 and 3): a static head keeps
// the frames its mask marks, a dynamic head keeps min(m, F_h) frames, so every
// offset is known on the host before any data is read and no call needs a
// device-to-host copy.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdint>
#include <initializer_list>
#include <mutex>
#include <string>

#include "fkv.h"
#include "fkv_launch.h"
#include "fkv_fp8.h"

static_assert(FKV_SCRATCH_BYTES == fkv::kScratchBytes,
              "fkv.h and fkv_launch.h must agree on the scratch size");

namespace fkv {
// calib.hip: `blocks` 256-thread workgroups, 8 x iters MFMAs per wave.
hipError_t launch_mfma_peak(float *sink, int blocks, int iters, hipStream_t s);
}  // namespace fkv

namespace {

thread_local std::string g_last_error;

fkv_status_t fail(fkv_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fkv_status_t ok() {
  g_last_error.clear();
  return FKV_OK;
}

int elt_bytes(int32_t dtype) { return dtype == FKV_BF16 ? 2 : 4; }

// The kernels move 16-byte pieces of every tensor and workspace they read or
// write, so those must start on a 16-byte boundary (NULL passes here; the
// NULL checks are separate).
fkv_status_t check_aligned(std::initializer_list<const void *> ptrs, const char *what) {
  for (const void *ptr : ptrs)
    if (reinterpret_cast<uintptr_t>(ptr) & 15u)
      return fail(FKV_ERR_SHAPE, "%s: a pointer is not 16-byte aligned", what);
  return FKV_OK;
}

// The query block and the plain window of a compression.
fkv_status_t check_inputs(const void *q, const void *k_cache, const void *v_cache) {
  if (!q || !k_cache || !v_cache) return fail(FKV_ERR_NULL, "q, k_cache or v_cache is NULL");
  return check_aligned({q, k_cache, v_cache}, "q, k_cache or v_cache");
}

float log2e_scale(const fkv_desc_t &d) {
  const float scale = d.scale != 0.f ? d.scale : 1.0f / std::sqrt((float)d.head_dim);
  return scale * 1.4426950408889634f;
}

fkv_status_t check_desc(const fkv_desc_t *d) {
  if (!d) return fail(FKV_ERR_NULL, "desc is NULL");
  if (d->dtype != FKV_BF16 && d->dtype != FKV_F32)
    return fail(FKV_ERR_DTYPE, "dtype %d is neither FKV_BF16 nor FKV_F32", d->dtype);
  if (d->dtype == FKV_BF16 && d->head_dim != 128)
    return fail(FKV_ERR_DTYPE, "bf16 needs head_dim 128 (got %d)", d->head_dim);
  if (d->dtype == FKV_F32 && d->head_dim != 64 && d->head_dim != 128)
    return fail(FKV_ERR_DTYPE, "fp32 needs head_dim 64 or 128 (got %d)", d->head_dim);
  if (d->num_heads < 1 || d->num_heads > fkv::kMaxHeads)
    return fail(FKV_ERR_SHAPE, "num_heads %d outside [1, %d]", d->num_heads, fkv::kMaxHeads);
  if (d->hist_frames < 0 || d->hist_frames > fkv::kMaxHistFrames)
    return fail(FKV_ERR_SHAPE, "hist_frames %d outside [0, %d]", d->hist_frames,
                fkv::kMaxHistFrames);
  if (d->cur_frames < 1 || d->cur_frames > fkv::kMaxCurFrames)
    return fail(FKV_ERR_SHAPE, "cur_frames %d outside [1, %d]", d->cur_frames, fkv::kMaxCurFrames);
  if (d->tokens_per_frame < 1)
    return fail(FKV_ERR_SHAPE, "tokens_per_frame %d < 1", d->tokens_per_frame);
  if (d->query_stride < 1) return fail(FKV_ERR_SHAPE, "query_stride %d < 1", d->query_stride);
  if (!std::isfinite(d->scale) || d->scale < 0.f)
    return fail(FKV_ERR_SHAPE, "scale must be finite and >= 0 (0 = 1/sqrt(D))");
  const int64_t n_win = (int64_t)(d->hist_frames + d->cur_frames) * d->tokens_per_frame;
  if (n_win >= (int64_t)1 << 31) return fail(FKV_ERR_SHAPE, "window of %lld tokens too long",
                                            (long long)n_win);
  // The kernels address K / V through buffer descriptors with 32-bit byte
  // ranges: one window tensor must stay below 4 GiB.
  const int64_t win_bytes = n_win * d->num_heads * d->head_dim * elt_bytes(d->dtype);
  if (win_bytes >= (int64_t)1 << 32)
    return fail(FKV_ERR_SHAPE, "window tensor of %lld bytes: 4 GiB or more is not supported",
                (long long)win_bytes);
  return FKV_OK;
}

struct Plan {
  int H, D, T, Fh, Fc, Ft, s, n_q, n_win, n_s, budget, n_dyn;
  int fh[fkv::kMaxHeads];  // history frames of each head (F_h for a plain window)
  int dyn_index[fkv::kMaxHeads];
  int dyn_heads[fkv::kMaxHeads];
  uint64_t static_bits[fkv::kMaxHeads];
  int32_t seg_off[fkv::kMaxHeads + 1];
  int32_t slot_off[fkv::kMaxHeads + 1];
  int64_t tok_off[fkv::kMaxHeads + 1];
  // Compaction jobs fixed before any score is known (static heads' kept
  // frames, every head's current chunk) and the rest (dynamic heads' kept
  // history frames), as prefix sums over heads.
  int32_t kept[fkv::kMaxHeads];
  int32_t n_hist_fixed[fkv::kMaxHeads];
  int32_t fixed_off[fkv::kMaxHeads + 1];
  int32_t dyn_slot_off[fkv::kMaxHeads + 1];
  size_t ws_lse_off, ws_slot_off, ws_bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// hist_frames: per-head history lengths (a rolling cache), or null for a
// plain window (every head has F_h).
fkv_status_t make_plan(const fkv_desc_t *d, const int32_t *hist_frames, const uint8_t *role,
                       const uint8_t *mask, int32_t budget_m, Plan *p) {
  fkv_status_t st = check_desc(d);
  if (st != FKV_OK) return st;
  if (!role) return fail(FKV_ERR_NULL, "head_role is NULL");
  if (budget_m < 0) return fail(FKV_ERR_BUDGET, "budget_m %d < 0", budget_m);
  p->H = d->num_heads;
  p->D = d->head_dim;
  p->T = d->tokens_per_frame;
  p->Fh = d->hist_frames;
  p->Fc = d->cur_frames;
  p->Ft = p->Fh + p->Fc;
  p->s = d->query_stride;
  p->n_q = p->Fc * p->T;
  p->n_win = p->Ft * p->T;
  p->n_s = (p->n_q + p->s - 1) / p->s;
  p->budget = budget_m;
  p->n_dyn = 0;
  bool any_static = false;
  for (int h = 0; h < p->H; ++h) {
    if (role[h] != FKV_STATIC && role[h] != FKV_DYNAMIC)
      return fail(FKV_ERR_SHAPE, "head_role[%d] = %d is neither static (0) nor dynamic (1)", h,
                  role[h]);
    const int fh = hist_frames ? hist_frames[h] : p->Fh;
    if (fh < 0 || fh > p->Fh)
      return fail(FKV_ERR_SHAPE, "hist_frames[%d] = %d outside [0, %d]", h, fh, p->Fh);
    p->fh[h] = fh;
    any_static |= role[h] == FKV_STATIC && fh > 0;
  }
  if (any_static && !mask)
    return fail(FKV_ERR_NULL, "static_keep_mask is NULL but static heads exist");
  p->seg_off[0] = 0;
  p->slot_off[0] = 0;
  p->tok_off[0] = 0;
  p->fixed_off[0] = 0;
  p->dyn_slot_off[0] = 0;
  for (int h = 0; h < p->H; ++h) {
    int kept;
    p->static_bits[h] = 0;
    p->dyn_index[h] = -1;
    if (role[h] == FKV_DYNAMIC) {
      // A dynamic head without history has nothing to score or keep.
      if (p->fh[h] > 0) {
        p->dyn_index[h] = p->n_dyn;
        p->dyn_heads[p->n_dyn++] = h;
      }
      kept = budget_m < p->fh[h] ? budget_m : p->fh[h];
    } else {
      uint64_t bits = 0;
      for (int f = 0; f < p->Fh; ++f) {
        if (!mask || !mask[(size_t)h * p->Fh + f]) continue;
        if (f >= p->fh[h])
          return fail(FKV_ERR_SHAPE,
                      "static_keep_mask[%d][%d] marks a frame beyond the head's %d history "
                      "frames", h, f, p->fh[h]);
        bits |= 1ull << f;
      }
      p->static_bits[h] = bits;
      kept = __builtin_popcountll(bits);
    }
    p->seg_off[h + 1] = p->seg_off[h] + kept;
    p->slot_off[h + 1] = p->slot_off[h] + kept + p->Fc;
    p->tok_off[h + 1] = p->tok_off[h] + (int64_t)(kept + p->Fc) * p->T;
    p->kept[h] = kept;
    p->n_hist_fixed[h] = role[h] == FKV_DYNAMIC ? 0 : kept;
    p->fixed_off[h + 1] = p->fixed_off[h] + p->n_hist_fixed[h] + p->Fc;
    p->dyn_slot_off[h + 1] = p->dyn_slot_off[h] + (p->dyn_index[h] >= 0 ? kept : 0);
  }
  for (int h = p->n_dyn; h < fkv::kMaxHeads; ++h) p->dyn_heads[h] = 0;
  for (int h = p->H; h < fkv::kMaxHeads; ++h) {
    p->dyn_index[h] = -1;
    p->static_bits[h] = 0;
    p->fh[h] = 0;
    p->kept[h] = 0;
    p->n_hist_fixed[h] = 0;
  }
  for (int h = p->H + 1; h <= fkv::kMaxHeads; ++h) {
    p->seg_off[h] = p->seg_off[p->H];
    p->slot_off[h] = p->slot_off[p->H];
    p->tok_off[h] = p->tok_off[p->H];
    p->fixed_off[h] = p->fixed_off[p->H];
    p->dyn_slot_off[h] = p->dyn_slot_off[p->H];
  }
  const size_t lse_bytes = p->n_dyn > 0 ? (size_t)p->n_dyn * p->n_s * p->Ft * sizeof(float) : 0;
  p->ws_lse_off = 0;
  p->ws_slot_off = align256(lse_bytes);
  p->ws_bytes = p->ws_slot_off + align256((size_t)p->slot_off[p->H] * sizeof(fkv::CopySlot));
  return FKV_OK;
}

fkv::WinView plain_window(const fkv_desc_t *d, const void *k, const void *v) {
  const int eb = elt_bytes(d->dtype);
  fkv::WinView w;
  w.hist_k = reinterpret_cast<const char *>(k);
  w.hist_v = reinterpret_cast<const char *>(v);
  w.hist_off = nullptr;
  w.tm_row_bytes = (int64_t)d->num_heads * d->head_dim * eb;
  w.row_bytes = d->head_dim * eb;
  const int64_t cur = (int64_t)d->hist_frames * d->tokens_per_frame * w.tm_row_bytes;
  w.cur_k = w.hist_k + cur;
  w.cur_v = w.hist_v + cur;
  return w;
}

fkv_status_t hip_fail(hipError_t e, const char *what) {
  return fail(FKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A second stream per device for the compaction jobs that do not depend on
// the scores, so that those copies (HBM-bound) run beside the scoring
// instead of after the selection.  Created on first use (non-blocking, the
// default priority); the fork and the join are events.  The device's mutex
// is held from the fork to the join, so calls from several host threads
// cannot interleave their events.
struct SideStream {
  std::mutex mu;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t copied = nullptr;  // after the fixed copies (fkv_compress_attend)
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];

// The current device's side stream, locked through *lock.
hipError_t side_stream(SideStream **out, std::unique_lock<std::mutex> *lock) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SideStream &ss = g_side[dev];
  *lock = std::unique_lock<std::mutex>(ss.mu);
  if (!ss.s) {
    hipStream_t st = nullptr;
    hipEvent_t ef = nullptr, ej = nullptr, ec = nullptr;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    // The events order two streams of one device and are never waited on by
    // the host: no timing, and no system-scope fence (the kernels' own
    // device-scope release and acquire make their writes visible).
    const unsigned flags = hipEventDisableTiming | hipEventDisableSystemFence;
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ef, flags);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ej, flags);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ec, flags);
    if (e != hipSuccess) {
      // Best-effort cleanup; the creation error is the one reported.
      if (ec) (void)hipEventDestroy(ec);
      if (ej) (void)hipEventDestroy(ej);
      if (ef) (void)hipEventDestroy(ef);
      if (st) (void)hipStreamDestroy(st);
      return e;
    }
    ss.s = st;
    ss.fork = ef;
    ss.join = ej;
    ss.copied = ec;
  }
  *out = &ss;
  return hipSuccess;
}

fkv_status_t attend_common(const fkv_desc_t *d, const void *q, const void *k, const void *v,
                           const int64_t *tok_off, void *out, void *workspace,
                           size_t workspace_bytes, void *stream) {
  const fkv_status_t st =
      check_aligned({q, k, v, out, workspace}, "q, k, v, out or the attention workspace");
  if (st != FKV_OK) return st;
  if (workspace && d->dtype == FKV_BF16) {
    const size_t need = fkv::attend_part_bytes();
    if (need == 0) return fail(FKV_ERR_HIP, "no HIP device to size the attention workspace for");
    if (workspace_bytes < need)
      return fail(FKV_ERR_WORKSPACE, "attention workspace of %zu bytes, %zu needed",
                  workspace_bytes, need);
  }
  fkv::AttendArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.tok_off = tok_off;
  a.kv_row_stride = (int64_t)d->num_heads * d->head_dim;
  a.dense_len = (d->hist_frames + d->cur_frames) * d->tokens_per_frame;
  a.n_q = d->cur_frames * d->tokens_per_frame;
  a.H = d->num_heads;
  a.D = d->head_dim;
  a.c = log2e_scale(*d);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  a.part = nullptr;
  a.n_wg = 0;
  a.n_sel = 0;
  hipError_t e = d->dtype == FKV_BF16 ? fkv::launch_attend_bf16(a, workspace, workspace_bytes, s)
                                      : fkv::launch_attend_f32(a, s);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  return ok();
}

// The query pointer and the output cache of a compression with plan p.
fkv_status_t check_compress_out(const Plan &p, const void *q, const fkv_ckv_t *out) {
  if (!q) return fail(FKV_ERR_NULL, "q is NULL");
  if (!out) return fail(FKV_ERR_NULL, "out (fkv_ckv_t) is NULL");
  if (!out->k || !out->v || !out->tok_off || !out->seg_off || (!out->seg_idx && p.Fh > 0))
    return fail(FKV_ERR_NULL, "a compressed-cache buffer (k, v, tok_off, seg_idx, seg_off) is NULL");
  const fkv_status_t st = check_aligned({q, out->k, out->v}, "q or the compressed cache's k, v");
  if (st != FKV_OK) return st;
  if (out->cap_tokens < p.tok_off[p.H])
    return fail(FKV_ERR_CAPACITY, "cap_tokens %lld < %lld rows needed",
                (long long)out->cap_tokens, (long long)p.tok_off[p.H]);
  return FKV_OK;
}

// Attention over the ragged cache `out` of the heads that have scored frames
// (scored = true) or of the others, with the plan's row offsets.
hipError_t attend_heads(const fkv_desc_t *d, const Plan &p, const void *q, const fkv_ckv_t *out,
                        void *attend_out, bool scored, hipStream_t s) {
  fkv::AttendArgs a;
  a.q = q;
  a.k = out->k;
  a.v = out->v;
  a.out = attend_out;
  a.tok_off = nullptr;
  a.kv_row_stride = d->head_dim;
  a.dense_len = 0;
  a.n_q = p.n_q;
  a.H = p.H;
  a.D = p.D;
  a.c = log2e_scale(*d);
  a.part = nullptr;
  a.n_wg = 0;
  a.n_sel = 0;
  for (int h = 0; h < p.H; ++h)
    if ((p.dyn_index[h] >= 0) == scored) a.sel[a.n_sel++] = h;
  for (int h = a.n_sel; h < fkv::kMaxHeads; ++h) a.sel[h] = 0;
  std::memcpy(a.host_off, p.tok_off, sizeof(a.host_off));
  if (a.n_sel == 0) return hipSuccess;
  return fkv::launch_attend_bf16_heads(a, s);
}

// Scoring, selection and compaction of one layer over the window `win`
// (plain or rolling) with the plan p.
// kv_scales (host [2 H]: K scales, then V scales) selects an e4m3 cache.
// side: copy the compaction jobs that do not depend on the scores on the
// device's side stream, beside the scoring (not with ev).
// attend_out (bf16, with side): also the attention of the compressed cache
// into attend_out [Nq, H, D], one workgroup per (head, 128-query tile): the
// heads whose copies are all fixed by the plan right after those copies on
// the side stream, the others after their copies on the caller's stream.
fkv_status_t compress_common(const fkv_desc_t *desc, const Plan &p, const void *q,
                             const fkv::WinView &win, const fkv_ckv_t *out, void *workspace,
                             size_t workspace_bytes, void *stream,
                             const float *kv_scales = nullptr, hipEvent_t *ev = nullptr,
                             bool side = false, void *attend_out = nullptr) {
  fkv_status_t st = check_compress_out(p, q, out);
  if (st != FKV_OK) return st;
  if (workspace_bytes < p.ws_bytes || (p.ws_bytes > 0 && !workspace))
    return fail(FKV_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                p.ws_bytes);
  st = check_aligned({workspace}, "workspace");
  if (st != FKV_OK) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = reinterpret_cast<char *>(workspace);
  float *lse = reinterpret_cast<float *>(ws + p.ws_lse_off);
  fkv::CopySlot *slots = reinterpret_cast<fkv::CopySlot *>(ws + p.ws_slot_off);
  const float c = log2e_scale(*desc);

  const bool split = side && !ev;
  SideStream *ss = nullptr;
  std::unique_lock<std::mutex> side_lock;
  // Joins the side stream into the caller's stream after the fork, before
  // the lock is released.  Without attend_out the join is made before the
  // dynamic heads' copies, with it at the end (the scored heads' attention
  // waits only for the fixed copies); both are checked.  On an early error
  // return the destructor still makes it, as a best effort, so that the
  // caller's stream never runs ahead of work already enqueued on the side
  // stream.
  struct Join {
    hipStream_t s = nullptr;
    hipEvent_t ev = nullptr;
    hipError_t now() {
      const hipError_t e = ev ? hipStreamWaitEvent(s, ev, 0) : hipSuccess;
      ev = nullptr;
      return e;
    }
    ~Join() { (void)now(); }
  } join;
  // Stage boundaries of fkv_compress_timed.
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };
  if (split) {
    // 0. fork point: the side stream starts from the caller's stream as it
    // stands before the scoring
    hipError_t e = side_stream(&ss, &side_lock);
    if (e != hipSuccess) return hip_fail(e, "side stream creation");
    e = hipEventRecord(ss->fork, s);
    if (e != hipSuccess) return hip_fail(e, "side stream fork");
  }
  if (hipError_t e = mark(0); e != hipSuccess) return hip_fail(e, "timing event");
  // 1. dynamic-head scoring: per (sampled query, frame) log-sum-exp
  hipError_t score_err = hipSuccess;
  if (p.n_dyn > 0) {
    fkv::ScoreArgs sa;
    sa.q = q;
    sa.win = win;
    sa.lse = lse;
    sa.H = p.H;
    sa.D = p.D;
    sa.T = p.T;
    sa.F_c = p.Fc;
    sa.F_tot = p.Ft;
    sa.n_s = p.n_s;
    sa.stride = p.s;
    sa.n_dyn = p.n_dyn;
    sa.n_qb = 0;
    sa.c = c;
    std::memcpy(sa.dyn_heads, p.dyn_heads, sizeof(sa.dyn_heads));
    std::memcpy(sa.fh, p.fh, sizeof(sa.fh));
    score_err = desc->dtype == FKV_BF16 ? fkv::launch_score_bf16(sa, s)
                                        : fkv::launch_score_f32(sa, s);
  }
  if (split) {
    // The score-independent copies on the side stream, enqueued after the
    // scoring so that the scoring workgroups are dispatched first and the
    // copies fill the remaining room.
    hipError_t e = hipStreamWaitEvent(ss->s, ss->fork, 0);
    if (e != hipSuccess) return hip_fail(e, "side stream fork");
    fkv::FixedCopyPlan cp;
    cp.win = win;
    cp.k_out = reinterpret_cast<char *>(out->k);
    cp.v_out = reinterpret_cast<char *>(out->v);
    cp.H = p.H;
    cp.T = p.T;
    cp.chunks = (p.T + fkv::kCompactRows - 1) / fkv::kCompactRows;
    std::memcpy(cp.fh, p.fh, sizeof(cp.fh));
    std::memcpy(cp.fixed_off_h, p.fixed_off, sizeof(cp.fixed_off_h));
    std::memcpy(cp.n_hist_fixed, p.n_hist_fixed, sizeof(cp.n_hist_fixed));
    std::memcpy(cp.kept, p.kept, sizeof(cp.kept));
    std::memcpy(cp.static_bits, p.static_bits, sizeof(cp.static_bits));
    std::memcpy(cp.tok_off_h, p.tok_off, sizeof(cp.tok_off_h));
    hipError_t el;
    if (kv_scales) {
      fkv::Fp8Scales sc;
      sc.D = p.D;
      for (int h = 0; h < fkv::kMaxHeads; ++h) {
        sc.k_scale[h] = h < p.H ? kv_scales[h] : 1.f;
        sc.v_scale[h] = h < p.H ? kv_scales[p.H + h] : 1.f;
      }
      el = fkv::launch_compact_fp8_fixed(cp, sc, ss->s);
    } else {
      el = fkv::launch_compact_fixed(cp, ss->s);
    }
    if (attend_out && el == hipSuccess) {
      // The heads with no scored frames are complete once the fixed copies
      // are: their attention starts here, beside the scoring and selection.
      e = hipEventRecord(ss->copied, ss->s);
      if (e != hipSuccess) el = e;
      if (el == hipSuccess) el = attend_heads(desc, p, q, out, attend_out, false, ss->s);
    }
    e = hipEventRecord(ss->join, ss->s);
    if (e != hipSuccess) return hip_fail(e, "side stream join");
    join.s = s;
    join.ev = ss->join;
    if (el != hipSuccess) return hip_fail(el, "side stream launch");
  }
  if (score_err != hipSuccess) return hip_fail(score_err, "scoring kernel launch");
  if (hipError_t e = mark(1); e != hipSuccess) return hip_fail(e, "timing event");
  // 2. selection, offsets and compaction slots
  {
    fkv::SelectArgs sa;
    sa.lse = p.n_dyn > 0 ? lse : nullptr;
    sa.seg_idx = out->seg_idx;
    sa.seg_off = out->seg_off;
    sa.tok_off = out->tok_off;
    sa.seg_score = p.Fh > 0 ? out->seg_score : nullptr;
    sa.slots = slots;
    sa.H = p.H;
    sa.T = p.T;
    sa.F_h = p.Fh;
    sa.F_c = p.Fc;
    sa.F_tot = p.Ft;
    sa.n_s = p.n_s;
    sa.budget = p.budget;
    sa.dyn_slots_only = split ? 1 : 0;
    std::memcpy(sa.fh, p.fh, sizeof(sa.fh));
    std::memcpy(sa.dyn_index, p.dyn_index, sizeof(sa.dyn_index));
    std::memcpy(sa.static_bits, p.static_bits, sizeof(sa.static_bits));
    std::memcpy(sa.seg_off_h, p.seg_off, sizeof(sa.seg_off_h));
    std::memcpy(sa.slot_off_h, split ? p.dyn_slot_off : p.slot_off, sizeof(sa.slot_off_h));
    std::memcpy(sa.tok_off_h, p.tok_off, sizeof(sa.tok_off_h));
    hipError_t e = fkv::launch_select(sa, s);
    if (e != hipSuccess) return hip_fail(e, "selection kernel launch");
  }
  if (hipError_t e = mark(2); e != hipSuccess) return hip_fail(e, "timing event");
  if (!attend_out) {
    const hipError_t e = join.now();
    if (e != hipSuccess) return hip_fail(e, "side stream join");
  }
  // 3. compaction
  if (kv_scales) {
    fkv::CompactFp8Args ca;
    ca.slots = slots;
    ca.win = win;
    ca.k_out = reinterpret_cast<uint8_t *>(out->k);
    ca.v_out = reinterpret_cast<uint8_t *>(out->v);
    ca.T = p.T;
    ca.chunks = (p.T + fkv::kCompactRows - 1) / fkv::kCompactRows;
    ca.D = p.D;
    std::memcpy(ca.fh, p.fh, sizeof(ca.fh));
    for (int h = 0; h < fkv::kMaxHeads; ++h) {
      ca.k_scale[h] = h < p.H ? kv_scales[h] : 1.f;
      ca.v_scale[h] = h < p.H ? kv_scales[p.H + h] : 1.f;
    }
    hipError_t e = fkv::launch_compact_fp8(ca, split ? p.dyn_slot_off[p.H] : p.slot_off[p.H], s);
    if (e != hipSuccess) return hip_fail(e, "quantizing compaction kernel launch");
  } else {
    fkv::CompactArgs ca;
    ca.slots = slots;
    ca.win = win;
    ca.k_out = reinterpret_cast<char *>(out->k);
    ca.v_out = reinterpret_cast<char *>(out->v);
    ca.out_tok_off = nullptr;
    ca.T = p.T;
    ca.F_c = p.Fc;
    ca.chunks = (p.T + fkv::kCompactRows - 1) / fkv::kCompactRows;
    std::memcpy(ca.fh, p.fh, sizeof(ca.fh));
    hipError_t e = fkv::launch_compact(ca, split ? p.dyn_slot_off[p.H] : p.slot_off[p.H], s);
    if (e != hipSuccess) return hip_fail(e, "compaction kernel launch");
  }
  if (hipError_t e = mark(3); e != hipSuccess) return hip_fail(e, "timing event");
  if (attend_out && split) {
    // 4. attention of the scored heads, whose current chunk the side stream
    // copied, then the join of the side stream's own attention
    hipError_t e = hipStreamWaitEvent(s, ss->copied, 0);
    if (e == hipSuccess) e = attend_heads(desc, p, q, out, attend_out, true, s);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    e = join.now();
    if (e != hipSuccess) return hip_fail(e, "side stream join");
  }
  return ok();
}

// ---- token-granular plan ---------------------------------------------------

struct TokenPlan {
  int H, D, T, Fh, Fc, n_q, n_hist, n_cur, sink_tok, recent_tok, cand_lo, cand_hi, n_cand;
  int budget, boundary, n_dyn, max_rows;
  int dyn_heads[fkv::kMaxHeads];
  int dyn_index[fkv::kMaxHeads];
  int64_t tok_off[fkv::kMaxHeads + 1];
  size_t ws_qsum_off, ws_phi_off, ws_src_off, ws_bytes;
};

// History tokens a static head keeps: the sink tokens and both ends of every
// aligned chunk, as a union of at most two intervals per chunk.
int64_t static_token_count(int n_hist, int chunk, int sink_tok, int L) {
  int64_t count = 0;
  for (int lo = 0; lo < n_hist; lo += chunk) {
    const int hi = lo + chunk < n_hist ? lo + chunk : n_hist;
    int e1 = lo + L < hi ? lo + L : hi;                       // [lo, e1): first L (and sink)
    const int sink_end = sink_tok < hi ? sink_tok : hi;
    if (sink_end > e1) e1 = sink_end;
    const int s2 = hi - L > lo ? hi - L : lo;                 // [s2, hi): last L
    const int overlap = e1 > s2 ? e1 - s2 : 0;
    count += (e1 - lo) + (hi - s2) - overlap;
  }
  return count;
}

fkv_status_t make_token_plan(const fkv_desc_t *d, const fkv_token_cfg_t *cfg,
                             const uint8_t *role, TokenPlan *p) {
  fkv_status_t st = check_desc(d);
  if (st != FKV_OK) return st;
  if (!cfg || !role) return fail(FKV_ERR_NULL, "cfg or head_role is NULL");
  if (cfg->sink_frames < 0 || cfg->recent_frames < 0 || cfg->boundary_tokens < 0)
    return fail(FKV_ERR_SHAPE, "sink_frames, recent_frames and boundary_tokens must be >= 0");
  if (cfg->budget_tokens < 0) return fail(FKV_ERR_BUDGET, "budget_tokens %d < 0",
                                          cfg->budget_tokens);
  p->H = d->num_heads;
  p->D = d->head_dim;
  p->T = d->tokens_per_frame;
  p->Fh = d->hist_frames;
  p->Fc = d->cur_frames;
  p->n_q = p->Fc * p->T;
  p->n_hist = p->Fh * p->T;
  p->n_cur = p->Fc * p->T;
  const int sink_f = cfg->sink_frames < p->Fh ? cfg->sink_frames : p->Fh;
  const int rest = p->Fh - sink_f;
  const int recent_f = cfg->recent_frames < rest ? cfg->recent_frames : rest;
  p->sink_tok = sink_f * p->T;
  p->recent_tok = recent_f * p->T;
  p->cand_lo = p->sink_tok;
  p->cand_hi = p->n_hist - p->recent_tok;
  p->n_cand = p->cand_hi - p->cand_lo;
  p->budget = cfg->budget_tokens;
  p->boundary = cfg->boundary_tokens;
  p->n_dyn = 0;
  p->max_rows = 0;
  p->tok_off[0] = 0;
  const int64_t dyn_kept = (int64_t)p->sink_tok + (p->budget < p->n_cand ? p->budget : p->n_cand) +
                           p->recent_tok;
  const int64_t st_kept = static_token_count(p->n_hist, p->Fc * p->T, p->sink_tok, p->boundary);
  for (int h = 0; h < p->H; ++h) {
    if (role[h] != FKV_STATIC && role[h] != FKV_DYNAMIC)
      return fail(FKV_ERR_SHAPE, "head_role[%d] = %d is neither static (0) nor dynamic (1)", h,
                  role[h]);
    p->dyn_index[h] = -1;
    if (role[h] == FKV_DYNAMIC) {
      p->dyn_index[h] = p->n_dyn;
      p->dyn_heads[p->n_dyn++] = h;
    }
    const int64_t rows = (role[h] == FKV_DYNAMIC ? dyn_kept : st_kept) + p->n_cur;
    p->tok_off[h + 1] = p->tok_off[h] + rows;
    if (rows > p->max_rows) p->max_rows = (int)rows;
  }
  for (int h = p->n_dyn; h < fkv::kMaxHeads; ++h) p->dyn_heads[h] = 0;
  for (int h = p->H; h < fkv::kMaxHeads; ++h) p->dyn_index[h] = -1;
  for (int h = p->H + 1; h <= fkv::kMaxHeads; ++h) p->tok_off[h] = p->tok_off[p->H];
  p->ws_qsum_off = 0;
  p->ws_phi_off = align256((size_t)p->n_dyn * p->D * sizeof(float));
  p->ws_src_off = p->ws_phi_off + align256((size_t)p->n_dyn * p->n_cand * sizeof(float));
  p->ws_bytes = p->ws_src_off + align256((size_t)p->tok_off[p->H] * sizeof(int32_t));
  return FKV_OK;
}

}  // namespace

extern "C" {

fkv_status_t fkv_plan(const fkv_desc_t *desc, const uint8_t *head_role,
                      const uint8_t *static_keep_mask, int32_t budget_m, int64_t *kept_tokens,
                      size_t *workspace_bytes) {
  Plan p;
  fkv_status_t st = make_plan(desc, nullptr, head_role, static_keep_mask, budget_m, &p);
  if (st != FKV_OK) return st;
  if (kept_tokens) *kept_tokens = p.tok_off[p.H];
  if (workspace_bytes) *workspace_bytes = p.ws_bytes;
  return ok();
}

fkv_status_t fkv_compress(const fkv_desc_t *desc, const void *q, const void *k_cache,
                          const void *v_cache, const uint8_t *head_role,
                          const uint8_t *static_keep_mask, int32_t budget_m, const fkv_ckv_t *out,
                          void *workspace, size_t workspace_bytes, void *stream) {
  Plan p;
  fkv_status_t st = make_plan(desc, nullptr, head_role, static_keep_mask, budget_m, &p);
  if (st != FKV_OK) return st;
  st = check_inputs(q, k_cache, v_cache);
  if (st != FKV_OK) return st;
  return compress_common(desc, p, q, plain_window(desc, k_cache, v_cache), out, workspace,
                         workspace_bytes, stream, nullptr, nullptr, true);
}

fkv_status_t fkv_compress_attend(const fkv_desc_t *desc, const void *q, const void *k_cache,
                                 const void *v_cache, const uint8_t *head_role,
                                 const uint8_t *static_keep_mask, int32_t budget_m,
                                 const fkv_ckv_t *out, void *workspace, size_t workspace_bytes,
                                 void *attend_out, void *attend_workspace,
                                 size_t attend_workspace_bytes, void *stream) {
  Plan p;
  fkv_status_t st = make_plan(desc, nullptr, head_role, static_keep_mask, budget_m, &p);
  if (st != FKV_OK) return st;
  st = check_inputs(q, k_cache, v_cache);
  if (st != FKV_OK) return st;
  if (!attend_out) return fail(FKV_ERR_NULL, "attend_out is NULL");
  st = check_aligned({attend_out, attend_workspace}, "attend_out or attend_workspace");
  if (st != FKV_OK) return st;
  st = check_compress_out(p, q, out);
  if (st != FKV_OK) return st;
  if (workspace_bytes < p.ws_bytes || (p.ws_bytes > 0 && !workspace))
    return fail(FKV_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                p.ws_bytes);
  if (attend_workspace && desc->dtype == FKV_BF16) {
    const size_t need = fkv::attend_part_bytes();
    if (need == 0) return fail(FKV_ERR_HIP, "no HIP device to size the attention workspace for");
    if (attend_workspace_bytes < need)
      return fail(FKV_ERR_WORKSPACE, "attention workspace of %zu bytes, %zu needed",
                  attend_workspace_bytes, need);
  }
  const fkv::WinView win = plain_window(desc, k_cache, v_cache);
  if (desc->dtype == FKV_BF16) {
    // With one workgroup per (head, query tile) the attention of the heads
    // without scored frames can start beside the scoring; the balanced
    // schedules run over all heads at once, after the compression.
    fkv::AttendArgs a;
    a.n_q = p.n_q;
    a.H = p.H;
    a.D = p.D;
    a.n_sel = 0;
    if (fkv::attend_bf16_schedule(a, attend_workspace, attend_workspace_bytes) == 0)
      return compress_common(desc, p, q, win, out, workspace, workspace_bytes, stream, nullptr,
                             nullptr, true, attend_out);
  }
  st = compress_common(desc, p, q, win, out, workspace, workspace_bytes, stream, nullptr,
                       nullptr, true);
  if (st != FKV_OK) return st;
  return attend_common(desc, q, out->k, out->v, out->tok_off, attend_out, attend_workspace,
                       attend_workspace_bytes, stream);
}

fkv_status_t fkv_compress_noalloc(const fkv_desc_t *desc, const void *q, const void *k_cache,
                                  const void *v_cache, const uint8_t *head_role,
                                  const uint8_t *static_keep_mask, int32_t budget_m,
                                  const fkv_ckv_t *out, void *stream) {
  Plan p;
  fkv_status_t st = make_plan(desc, nullptr, head_role, static_keep_mask, budget_m, &p);
  if (st != FKV_OK) return st;
  st = check_inputs(q, k_cache, v_cache);
  if (st != FKV_OK) return st;
  st = check_compress_out(p, q, out);
  if (st != FKV_OK) return st;
  if (p.ws_bytes > fkv::kScratchBytes)
    return fail(FKV_ERR_WORKSPACE,
                "this layer needs %zu bytes of workspace, more than the %zu bytes of the "
                "library's scratch memory; use fkv_compress with a caller workspace",
                p.ws_bytes, fkv::kScratchBytes);
  void *scratch = nullptr;
  if (p.ws_bytes > 0) {
    const hipError_t e = fkv::scratch_address(&scratch);
    if (e != hipSuccess) return hip_fail(e, "scratch memory address");
  }
  return compress_common(desc, p, q, plain_window(desc, k_cache, v_cache), out, scratch,
                         fkv::kScratchBytes, stream);
}

namespace {
fkv_status_t check_scales(const fkv_desc_t *d, const float *sc, int n, const char *what) {
  if (d->dtype != FKV_BF16) return fail(FKV_ERR_DTYPE, "the fp8 cache needs bf16 inputs");
  if (!sc) return fail(FKV_ERR_NULL, "%s is NULL", what);
  for (int i = 0; i < n; ++i)
    if (!(sc[i] > 0.f) || !std::isfinite(sc[i]))
      return fail(FKV_ERR_SHAPE, "%s[%d] = %g is not a positive finite scale", what, i,
                  (double)sc[i]);
  return FKV_OK;
}
}  // namespace

fkv_status_t fkv_compress_fp8(const fkv_desc_t *desc, const void *q, const void *k_cache,
                              const void *v_cache, const uint8_t *head_role,
                              const uint8_t *static_keep_mask, int32_t budget_m,
                              const float *kv_scales, const fkv_ckv_t *out, void *workspace,
                              size_t workspace_bytes, void *stream) {
  Plan p;
  fkv_status_t st = make_plan(desc, nullptr, head_role, static_keep_mask, budget_m, &p);
  if (st != FKV_OK) return st;
  st = check_scales(desc, kv_scales, 2 * desc->num_heads, "kv_scales");
  if (st != FKV_OK) return st;
  st = check_inputs(q, k_cache, v_cache);
  if (st != FKV_OK) return st;
  return compress_common(desc, p, q, plain_window(desc, k_cache, v_cache), out, workspace,
                         workspace_bytes, stream, kv_scales, nullptr, true);
}

fkv_status_t fkv_attend_fp8(const fkv_desc_t *desc, const void *q, const fkv_ckv_t *ckv,
                            const float *scales, void *out, void *workspace,
                            size_t workspace_bytes, void *stream) {
  fkv_status_t st = check_desc(desc);
  if (st != FKV_OK) return st;
  st = check_scales(desc, scales, 3 * desc->num_heads, "scales");
  if (st != FKV_OK) return st;
  if (!q || !out) return fail(FKV_ERR_NULL, "q or out is NULL");
  if (!ckv || !ckv->k || !ckv->v || !ckv->tok_off)
    return fail(FKV_ERR_NULL, "compressed cache (k, v, tok_off) is NULL");
  st = check_aligned({q, out, ckv->k, ckv->v, workspace},
                     "q, out, the cache's k, v or the attention workspace");
  if (st != FKV_OK) return st;
  if (workspace) {
    const size_t need = fkv::attend_part_bytes();
    if (need == 0) return fail(FKV_ERR_HIP, "no HIP device to size the attention workspace for");
    if (workspace_bytes < need)
      return fail(FKV_ERR_WORKSPACE, "attention workspace of %zu bytes, %zu needed",
                  workspace_bytes, need);
  }
  fkv::AttendFp8Args a;
  a.q = q;
  a.k = reinterpret_cast<const uint8_t *>(ckv->k);
  a.v = reinterpret_cast<const uint8_t *>(ckv->v);
  a.out = out;
  a.tok_off = ckv->tok_off;
  a.n_q = desc->cur_frames * desc->tokens_per_frame;
  a.H = desc->num_heads;
  a.c = log2e_scale(*desc);
  const int H = desc->num_heads;
  for (int h = 0; h < fkv::kMaxHeads; ++h) {
    a.q_scale[h] = h < H ? scales[h] : 1.f;
    a.k_scale[h] = h < H ? scales[H + h] : 1.f;
    a.v_scale[h] = h < H ? scales[2 * H + h] : 1.f;
  }
  hipError_t e = fkv::launch_attend_fp8(a, workspace, workspace ? workspace_bytes : 0,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 attention kernel launch");
  return ok();
}

fkv_status_t fkv_compress_timed(const fkv_desc_t *desc, const void *q, const void *k_cache,
                                const void *v_cache, const uint8_t *head_role,
                                const uint8_t *static_keep_mask, int32_t budget_m,
                                const fkv_ckv_t *out, void *workspace, size_t workspace_bytes,
                                void *stream, float *ms) {
  Plan p;
  fkv_status_t st = make_plan(desc, nullptr, head_role, static_keep_mask, budget_m, &p);
  if (st != FKV_OK) return st;
  st = check_inputs(q, k_cache, v_cache);
  if (st != FKV_OK) return st;
  if (!ms) return fail(FKV_ERR_NULL, "ms is NULL");
  hipEvent_t ev[4] = {};
  for (int i = 0; i < 4; ++i) {
    const hipError_t e = hipEventCreate(&ev[i]);
    if (e != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
      return hip_fail(e, "event creation");
    }
  }
  st = compress_common(desc, p, q, plain_window(desc, k_cache, v_cache), out, workspace,
                       workspace_bytes, stream, nullptr, ev);
  hipError_t e = st == FKV_OK ? hipEventSynchronize(ev[3]) : hipSuccess;
  for (int i = 0; st == FKV_OK && e == hipSuccess && i < 3; ++i)
    e = hipEventElapsedTime(&ms[i], ev[i], ev[i + 1]);
  // No scoring kernel runs without dynamic heads (the two events around the
  // empty stage would only time their own recording).
  if (st == FKV_OK && e == hipSuccess && p.n_dyn == 0) ms[0] = 0.f;
  for (int i = 0; i < 4; ++i) (void)hipEventDestroy(ev[i]);
  if (st != FKV_OK) return st;
  if (e != hipSuccess) return hip_fail(e, "event timing");
  return ok();
}

fkv_status_t fkv_plan_ragged(const fkv_desc_t *desc, const int32_t *hist_frames,
                             const uint8_t *head_role, const uint8_t *static_keep_mask,
                             int32_t budget_m, int64_t *kept_tokens, size_t *workspace_bytes) {
  if (!hist_frames) return fail(FKV_ERR_NULL, "hist_frames is NULL");
  Plan p;
  fkv_status_t st = make_plan(desc, hist_frames, head_role, static_keep_mask, budget_m, &p);
  if (st != FKV_OK) return st;
  if (kept_tokens) *kept_tokens = p.tok_off[p.H];
  if (workspace_bytes) *workspace_bytes = p.ws_bytes;
  return ok();
}

fkv_status_t fkv_compress_ragged(const fkv_desc_t *desc, const void *q, const fkv_ckv_t *hist,
                                 const int32_t *hist_frames, const void *cur_k,
                                 const void *cur_v, const uint8_t *head_role,
                                 const uint8_t *static_keep_mask, int32_t budget_m,
                                 const fkv_ckv_t *out, void *workspace, size_t workspace_bytes,
                                 void *stream) {
  if (!hist_frames) return fail(FKV_ERR_NULL, "hist_frames is NULL");
  Plan p;
  fkv_status_t st = make_plan(desc, hist_frames, head_role, static_keep_mask, budget_m, &p);
  if (st != FKV_OK) return st;
  if (!hist || !hist->k || !hist->v || !hist->tok_off)
    return fail(FKV_ERR_NULL, "history cache (k, v, tok_off) is NULL");
  if (!cur_k || !cur_v) return fail(FKV_ERR_NULL, "cur_k or cur_v is NULL");
  st = check_aligned({hist->k, hist->v, cur_k, cur_v}, "the history's k, v, cur_k or cur_v");
  if (st != FKV_OK) return st;
  if (out && (out->k == hist->k || out->v == hist->v || out->tok_off == hist->tok_off))
    return fail(FKV_ERR_SHAPE, "out must not share buffers with the history cache");
  fkv::WinView win = plain_window(desc, hist->k, hist->v);
  win.hist_off = hist->tok_off;
  win.cur_k = reinterpret_cast<const char *>(cur_k);
  win.cur_v = reinterpret_cast<const char *>(cur_v);
  return compress_common(desc, p, q, win, out, workspace, workspace_bytes, stream, nullptr,
                         nullptr, true);
}

fkv_status_t fkv_refresh_current(const fkv_desc_t *desc, const void *cur_k, const void *cur_v,
                                 const fkv_ckv_t *ckv, void *stream) {
  fkv_status_t st = check_desc(desc);
  if (st != FKV_OK) return st;
  if (!cur_k || !cur_v) return fail(FKV_ERR_NULL, "cur_k or cur_v is NULL");
  if (!ckv || !ckv->k || !ckv->v || !ckv->tok_off)
    return fail(FKV_ERR_NULL, "compressed cache (k, v, tok_off) is NULL");
  st = check_aligned({cur_k, cur_v, ckv->k, ckv->v}, "cur_k, cur_v or the cache's k, v");
  if (st != FKV_OK) return st;
  fkv::CompactArgs ca;
  ca.slots = nullptr;
  ca.win = plain_window(desc, nullptr, nullptr);
  ca.win.cur_k = reinterpret_cast<const char *>(cur_k);
  ca.win.cur_v = reinterpret_cast<const char *>(cur_v);
  ca.k_out = reinterpret_cast<char *>(ckv->k);
  ca.v_out = reinterpret_cast<char *>(ckv->v);
  ca.out_tok_off = ckv->tok_off;
  ca.T = desc->tokens_per_frame;
  ca.F_c = desc->cur_frames;
  ca.chunks = (ca.T + fkv::kCompactRows - 1) / fkv::kCompactRows;
  std::memset(ca.fh, 0, sizeof(ca.fh));  // every source frame is a current-chunk frame
  hipError_t e = fkv::launch_compact(ca, desc->num_heads * desc->cur_frames,
                                     reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "compaction kernel launch");
  return ok();
}

fkv_status_t fkv_roll_static_mask(int32_t n_frames, const int32_t *frame_ids,
                                  int32_t cur_frames, int32_t cap, uint8_t *mask) {
  if (n_frames < 0 || n_frames > fkv::kMaxHistFrames)
    return fail(FKV_ERR_SHAPE, "n_frames %d outside [0, %d]", n_frames, fkv::kMaxHistFrames);
  if (cur_frames < 1) return fail(FKV_ERR_SHAPE, "cur_frames %d < 1", cur_frames);
  if (cap < 0) return fail(FKV_ERR_SHAPE, "cap %d < 0", cap);
  if (n_frames > 0 && (!frame_ids || !mask)) return fail(FKV_ERR_NULL, "frame_ids or mask is NULL");
  int kept = 0;
  for (int i = 0; i < n_frames; ++i) {
    const int32_t id = frame_ids[i];
    if (id < 0) return fail(FKV_ERR_SHAPE, "frame_ids[%d] = %d < 0", i, id);
    const int32_t pos = id % cur_frames;
    mask[i] = (id == 0 || pos == 0 || pos == cur_frames - 1) ? 1 : 0;
    kept += mask[i];
  }
  // Over the cap: drop the oldest kept frames that are not the sink.
  for (int i = 0; i < n_frames && kept > cap; ++i) {
    if (mask[i] && frame_ids[i] != 0) {
      mask[i] = 0;
      --kept;
    }
  }
  // Only sinks left above the cap: drop the oldest of them too.
  for (int i = 0; i < n_frames && kept > cap; ++i) {
    if (mask[i]) {
      mask[i] = 0;
      --kept;
    }
  }
  return ok();
}

fkv_status_t fkv_plan_tokens(const fkv_desc_t *desc, const fkv_token_cfg_t *cfg,
                             const uint8_t *head_role, int64_t *kept_tokens,
                             size_t *workspace_bytes) {
  TokenPlan p;
  fkv_status_t st = make_token_plan(desc, cfg, head_role, &p);
  if (st != FKV_OK) return st;
  if (kept_tokens) *kept_tokens = p.tok_off[p.H];
  if (workspace_bytes) *workspace_bytes = p.ws_bytes;
  return ok();
}

fkv_status_t fkv_compress_tokens(const fkv_desc_t *desc, const fkv_token_cfg_t *cfg,
                                 const void *q, const void *k_cache, const void *v_cache,
                                 const uint8_t *head_role, const fkv_ckv_t *out,
                                 int32_t *row_src, void *workspace, size_t workspace_bytes,
                                 void *stream) {
  TokenPlan p;
  fkv_status_t st = make_token_plan(desc, cfg, head_role, &p);
  if (st != FKV_OK) return st;
  st = check_inputs(q, k_cache, v_cache);
  if (st != FKV_OK) return st;
  if (!out || !out->k || !out->v || !out->tok_off)
    return fail(FKV_ERR_NULL, "a compressed-cache buffer (k, v, tok_off) is NULL");
  if (out->cap_tokens < p.tok_off[p.H])
    return fail(FKV_ERR_CAPACITY, "cap_tokens %lld < %lld rows needed",
                (long long)out->cap_tokens, (long long)p.tok_off[p.H]);
  st = check_aligned({out->k, out->v}, "the compressed cache's k, v");
  if (st != FKV_OK) return st;
  if (!workspace || workspace_bytes < p.ws_bytes)
    return fail(FKV_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                p.ws_bytes);
  st = check_aligned({workspace}, "workspace");
  if (st != FKV_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // The plan's offsets reach the device as kernel arguments; the selection
  // kernel writes them to out->tok_off.
  char *ws = reinterpret_cast<char *>(workspace);
  fkv::TokenArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.k_out = reinterpret_cast<char *>(out->k);
  a.v_out = reinterpret_cast<char *>(out->v);
  a.src = row_src ? row_src : reinterpret_cast<int32_t *>(ws + p.ws_src_off);
  a.qsum = reinterpret_cast<float *>(ws + p.ws_qsum_off);
  a.phi = reinterpret_cast<float *>(ws + p.ws_phi_off);
  a.H = p.H;
  a.D = p.D;
  a.elt = elt_bytes(desc->dtype);
  a.T = p.T;
  a.F_c = p.Fc;
  a.n_q = p.n_q;
  a.stride = desc->query_stride;
  a.n_hist = p.n_hist;
  a.n_cur = p.n_cur;
  a.sink_tok = p.sink_tok;
  a.recent_tok = p.recent_tok;
  a.cand_lo = p.cand_lo;
  a.cand_hi = p.cand_hi;
  a.n_cand = p.n_cand;
  a.budget = p.budget;
  a.boundary = p.boundary;
  a.n_dyn = p.n_dyn;
  a.max_rows = p.max_rows;
  a.tok_off_out = out->tok_off;
  std::memcpy(a.dyn_heads, p.dyn_heads, sizeof(a.dyn_heads));
  std::memcpy(a.dyn_index, p.dyn_index, sizeof(a.dyn_index));
  std::memcpy(a.tok_off_h, p.tok_off, sizeof(a.tok_off_h));
  hipError_t e = fkv::launch_tokens(a, s);
  if (e != hipSuccess) return hip_fail(e, "token compression kernel launch");
  return ok();
}

fkv_status_t fkv_profile_workspace(const fkv_desc_t *desc, size_t *workspace_bytes) {
  fkv_status_t st = check_desc(desc);
  if (st != FKV_OK) return st;
  if (!workspace_bytes) return fail(FKV_ERR_NULL, "workspace_bytes is NULL");
  const int64_t n_q = (int64_t)desc->cur_frames * desc->tokens_per_frame;
  const int64_t n_s = (n_q + desc->query_stride - 1) / desc->query_stride;
  *workspace_bytes = (size_t)desc->num_heads * n_s * (desc->hist_frames + desc->cur_frames) *
                     sizeof(float);
  return ok();
}

fkv_status_t fkv_profile_heads(const fkv_desc_t *desc, const void *q, const void *k_cache,
                               float *mass_accum, void *workspace, size_t workspace_bytes,
                               void *stream) {
  fkv_status_t st = check_desc(desc);
  if (st != FKV_OK) return st;
  if (!q || !k_cache || !mass_accum) return fail(FKV_ERR_NULL, "q, k_cache or mass_accum is NULL");
  st = check_aligned({q, k_cache, workspace}, "q, k_cache or workspace");
  if (st != FKV_OK) return st;
  size_t need = 0;
  fkv_profile_workspace(desc, &need);
  if (!workspace || workspace_bytes < need)
    return fail(FKV_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int H = desc->num_heads, Ft = desc->hist_frames + desc->cur_frames;
  const int n_q = desc->cur_frames * desc->tokens_per_frame;
  fkv::ScoreArgs sa;
  sa.q = q;
  sa.win = plain_window(desc, k_cache, k_cache);
  sa.lse = reinterpret_cast<float *>(workspace);
  sa.H = H;
  sa.D = desc->head_dim;
  sa.T = desc->tokens_per_frame;
  sa.F_c = desc->cur_frames;
  sa.F_tot = Ft;
  sa.n_s = (n_q + desc->query_stride - 1) / desc->query_stride;
  sa.stride = desc->query_stride;
  sa.n_dyn = H;
  sa.n_qb = 0;
  sa.c = log2e_scale(*desc);
  for (int h = 0; h < fkv::kMaxHeads; ++h) {
    sa.dyn_heads[h] = h < H ? h : 0;
    sa.fh[h] = desc->hist_frames;
  }
  hipError_t e = desc->dtype == FKV_BF16 ? fkv::launch_score_bf16(sa, s)
                                         : fkv::launch_score_f32(sa, s);
  if (e != hipSuccess) return hip_fail(e, "scoring kernel launch");
  fkv::ProfileArgs pa;
  pa.lse = sa.lse;
  pa.out = mass_accum;
  pa.H = H;
  pa.F_tot = Ft;
  pa.n_s = sa.n_s;
  e = fkv::launch_profile(pa, s);
  if (e != hipSuccess) return hip_fail(e, "profiling kernel launch");
  return ok();
}

fkv_status_t fkv_classify_heads(const fkv_desc_t *desc, const float *mass_sum, int32_t n_calls,
                                float threshold, uint8_t *head_role, uint8_t *static_keep_mask,
                                float *discontinuity) {
  fkv_status_t st = check_desc(desc);
  if (st != FKV_OK) return st;
  if (!mass_sum || !head_role || (!static_keep_mask && desc->hist_frames > 0))
    return fail(FKV_ERR_NULL, "mass_sum, head_role or static_keep_mask is NULL");
  if (n_calls < 1) return fail(FKV_ERR_SHAPE, "n_calls %d < 1", n_calls);
  const int H = desc->num_heads, Fh = desc->hist_frames, Fc = desc->cur_frames;
  const int Ft = Fh + Fc;
  for (int h = 0; h < H; ++h) {
    const float *row = mass_sum + (size_t)h * Ft;
    double b_sum = 0, i_sum = 0;
    int b_n = 0, i_n = 0;
    for (int f = 0; f < Ft; ++f) {
      const int pos = f % Fc;
      const bool boundary = f == 0 || pos == 0 || pos == Fc - 1;
      const double m = (double)row[f] / n_calls;
      if (boundary) {
        b_sum += m;
        ++b_n;
      } else {
        i_sum += m;
        ++i_n;
      }
    }
    double disc = std::nan("");
    if (b_n > 0 && i_n > 0 && i_sum > 0) disc = (b_sum / b_n) / (i_sum / i_n);
    if (discontinuity) discontinuity[h] = (float)disc;
    const bool is_static = disc >= (double)threshold;  // false for NaN
    head_role[h] = is_static ? FKV_STATIC : FKV_DYNAMIC;
    for (int f = 0; f < Fh; ++f)
      static_keep_mask[(size_t)h * Fh + f] =
          is_static && (double)row[f] / n_calls >= 1.0 / Ft ? 1 : 0;
  }
  return ok();
}

fkv_status_t fkv_attend_workspace(const fkv_desc_t *desc, size_t *workspace_bytes) {
  fkv_status_t st = check_desc(desc);
  if (st != FKV_OK) return st;
  if (!workspace_bytes) return fail(FKV_ERR_NULL, "workspace_bytes is NULL");
  *workspace_bytes = 0;
  if (desc->dtype != FKV_BF16) return ok();
  const size_t need = fkv::attend_part_bytes();
  if (need == 0) return fail(FKV_ERR_HIP, "no HIP device to size the attention workspace for");
  *workspace_bytes = need;
  return ok();
}

fkv_status_t fkv_attend(const fkv_desc_t *desc, const void *q, const fkv_ckv_t *ckv, void *out,
                        void *workspace, size_t workspace_bytes, void *stream) {
  fkv_status_t st = check_desc(desc);
  if (st != FKV_OK) return st;
  if (!q || !out) return fail(FKV_ERR_NULL, "q or out is NULL");
  if (!ckv || !ckv->k || !ckv->v || !ckv->tok_off)
    return fail(FKV_ERR_NULL, "compressed cache (k, v, tok_off) is NULL");
  return attend_common(desc, q, ckv->k, ckv->v, ckv->tok_off, out, workspace, workspace_bytes,
                       stream);
}

fkv_status_t fkv_attend_dense(const fkv_desc_t *desc, const void *q, const void *k_cache,
                              const void *v_cache, void *out, void *workspace,
                              size_t workspace_bytes, void *stream) {
  fkv_status_t st = check_desc(desc);
  if (st != FKV_OK) return st;
  if (!q || !k_cache || !v_cache || !out)
    return fail(FKV_ERR_NULL, "q, k_cache, v_cache or out is NULL");
  return attend_common(desc, q, k_cache, v_cache, nullptr, out, workspace, workspace_bytes,
                       stream);
}

fkv_status_t fkv_mfma_peak(int32_t iters, float *sink, double *tflops) {
  if (!sink || !tflops) return fail(FKV_ERR_NULL, "sink or tflops is NULL");
  if (iters < 1) return fail(FKV_ERR_SHAPE, "iters %d < 1", iters);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  hipEvent_t ev[2] = {};
  if ((e = hipEventCreate(&ev[0])) != hipSuccess) return hip_fail(e, "event creation");
  if ((e = hipEventCreate(&ev[1])) != hipSuccess) {
    (void)hipEventDestroy(ev[0]);
    return hip_fail(e, "event creation");
  }
  const int blocks = 2 * cus;
  e = fkv::launch_mfma_peak(sink, blocks, 10, nullptr);  // warm-up
  if (e == hipSuccess) e = hipEventRecord(ev[0], nullptr);
  if (e == hipSuccess) e = fkv::launch_mfma_peak(sink, blocks, iters, nullptr);
  if (e == hipSuccess) e = hipEventRecord(ev[1], nullptr);
  if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  if (e != hipSuccess) return hip_fail(e, "MFMA calibration");
  // 4 waves per workgroup, 8 MFMAs of 32 x 32 x 16 (2 FLOP each) per iteration
  const double flop = (double)blocks * 4 * 8 * iters * 2.0 * 32 * 32 * 16;
  *tflops = flop / (ms * 1e-3) / 1e12;
  return ok();
}

const char *fkv_status_str(fkv_status_t status) {
  switch (status) {
    case FKV_OK: return "ok";
    case FKV_ERR_NULL: return "null pointer";
    case FKV_ERR_SHAPE: return "bad shape";
    case FKV_ERR_DTYPE: return "unsupported dtype / head dim";
    case FKV_ERR_BUDGET: return "negative budget";
    case FKV_ERR_CAPACITY: return "compressed cache too small";
    case FKV_ERR_WORKSPACE: return "workspace too small";
    case FKV_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *fkv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
