/*
 * fkv.h -- C ABI of libfkv.so: the per-layer hot path of Forcing-KV hybrid
 * head-wise KV-cache compression on AMD Instinct MI355X (gfx950).
 *
 * Sources for what each call computes (pages on the method):
 *   [S] "Forcing-KV：面向高效自回归视频扩散模型的混合KV缓存压缩" (ai-feeds.com
 *       summary of arXiv 2605.09681), section 方法 (Method): 输入与整体流程,
 *       关键模块 2 (static structural pruning), 关键模块 3 (dynamic similarity
 *       pruning), 输出与工程收益 (the compressed KV replaces the cache in the
 *       layer's attention); section 行业影响 › 与现有产品/工作流的接口 (a
 *       plug-in applied per attention layer at every denoising step, head
 *       labels produced offline once).
 *   [A] "Forcing-KV: Hybrid KV Cache Compression for Efficient Autoregressive
 *       Video Diffusion Models" (tomesphere.com), Abstract.
 *
 * Shapes and layouts (all tensors contiguous, row-major, in device memory
 * owned by the caller; T = tokens per latent frame, F_h history frames, F_c
 * current-chunk frames, H heads, D head dim):
 *   q        [Nq,    H, D]   Nq    = F_c * T        current chunk's queries
 *   k_cache  [N_win, H, D]   N_win = (F_h + F_c) * T
 *   v_cache  [N_win, H, D]   frames oldest first; the current chunk is last
 *   out      [Nq,    H, D]   same dtype as q
 * Element type: bf16 with D = 128, or fp32 with D = 64 or 128.
 * Limits: 1 <= H <= 64, 0 <= F_h <= 64, 1 <= F_c <= 8, 1 <= T, s >= 1,
 *         N_win < 2^31, each window tensor (N_win * H * D elements) below
 *         4 GiB; element offsets are computed in 64 bits.
 * Alignment: the kernels move 16-byte pieces, so every tensor (q, k_cache,
 *         v_cache, out, the compressed cache's k and v, cur_k, cur_v) and
 *         every workspace must start on a 16-byte boundary, else
 *         FKV_ERR_SHAPE; offset and index arrays need only their natural
 *         alignment.
 *
 * Threading and streams: calls are stateless apart from the thread-local
 * error string (and the scratch array of fkv_compress_noalloc); every device
 * operation is enqueued on the given stream (a hipStream_t passed as void*,
 * NULL = the default stream) and no call waits for the device.  The one
 * exception to a single stream: fkv_compress, fkv_compress_ragged,
 * fkv_compress_fp8 and fkv_compress_attend run the copies that do not depend
 * on the scores (and fkv_compress_attend some of the attention) on a second
 * stream of the library (one per device, non-blocking, default priority,
 * created with three events on the first such call and kept until the
 * process ends), forked from the given stream by an event before the scoring
 * and joined back into it by event waits before the call returns, so that
 * to the caller the call is still ordered on its stream like a single kernel
 * sequence.  Calls from several host threads
 * are serialised on that stream's per-device lock while they enqueue.  The
 * library allocates no device memory.
 *
 * Errors: argument errors are detected on the host before any HIP call and
 * returned as a status; a failed kernel launch returns FKV_ERR_HIP.  Faults
 * inside kernels surface at the caller's next synchronisation.  The text of
 * the last error on the calling thread is returned by fkv_last_error().
 */
#ifndef FKV_H
#define FKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FKV_OK = 0,
  FKV_ERR_NULL = 1,       /* a required pointer is NULL                        */
  FKV_ERR_SHAPE = 2,      /* a size is out of range or inconsistent            */
  FKV_ERR_DTYPE = 3,      /* unsupported element type / head dim combination   */
  FKV_ERR_BUDGET = 4,     /* budget_m < 0                                      */
  FKV_ERR_CAPACITY = 5,   /* compressed buffers too small for the kept rows    */
  FKV_ERR_WORKSPACE = 6,  /* workspace smaller than fkv_plan's figure          */
  FKV_ERR_HIP = 7         /* a HIP runtime call or kernel launch failed        */
} fkv_status_t;

typedef enum { FKV_BF16 = 0, FKV_F32 = 1 } fkv_dtype_t;

/* Head roles, produced by offline profiling ([S] 关键模块 1). */
typedef enum { FKV_STATIC = 0, FKV_DYNAMIC = 1 } fkv_role_t;

/* Problem description shared by every call. */
typedef struct fkv_desc {
  int32_t num_heads;        /* H                                              */
  int32_t head_dim;         /* D                                              */
  int32_t tokens_per_frame; /* T                                              */
  int32_t hist_frames;      /* F_h: history frames in the window              */
  int32_t cur_frames;       /* F_c: frames of the current chunk (queries)     */
  int32_t query_stride;     /* s: dynamic scoring uses queries 0, s, 2s, ...  */
  float scale;              /* logit scale; 0 selects 1/sqrt(D)               */
  int32_t dtype;            /* fkv_dtype_t of q, k_cache, v_cache, ckv, out   */
} fkv_desc_t;

/* The compressed cache of one layer ([S] 输出与工程收益): ragged, head-major.
 * Head h owns rows [tok_off[h], tok_off[h+1]) of k and v: the T rows of each
 * kept history frame in ascending frame order, then the T rows of each
 * current-chunk frame.  All pointers are caller-owned device memory. */
typedef struct fkv_ckv {
  void *k;             /* [cap_tokens, D] dtype                                */
  void *v;             /* [cap_tokens, D] dtype                                */
  int64_t *tok_off;    /* [H + 1]                                              */
  int32_t *seg_idx;    /* [H * F_h] kept history frames; head h's are
                          seg_idx[seg_off[h] .. seg_off[h+1]), ascending       */
  int32_t *seg_off;    /* [H + 1]                                              */
  float *seg_score;    /* [H * F_h] or NULL: score of every history frame of
                          every head (mean softmax mass); NaN for static heads */
  int64_t cap_tokens;  /* rows available in k and v                            */
} fkv_ckv_t;

/* Host-only planning ([S] 关键模块 2: a static head's reduction is fixed in
 * size once profiling has frozen its pattern; 关键模块 3: a dynamic head keeps
 * a fixed number of top segments).  The kept counts therefore depend only on
 * the roles, the static mask and the budget, so the compressed size is known
 * before any data is read.  head_role [H] and static_keep_mask [H * F_h]
 * (row-major; rows of dynamic heads ignored) are host arrays.  Writes the
 * rows the compressed cache needs (tok_off[H]) to *kept_tokens and the
 * workspace bytes fkv_compress needs to *workspace_bytes.  Either output pointer may be NULL.
 * A budget above F_h keeps every history frame of a dynamic head. */
fkv_status_t fkv_plan(const fkv_desc_t *desc, const uint8_t *head_role,
                      const uint8_t *static_keep_mask, int32_t budget_m,
                      int64_t *kept_tokens, size_t *workspace_bytes);

/* Compression of one layer ([S] 关键模块 2 and 3; [A]):
 *  - static heads keep the history frames their mask row marks;
 *  - dynamic heads score each history frame by the softmax attention mass
 *    it receives (softmax over the whole window, current chunk included,
 *    scale * q.k logits) averaged over the strided query sample, and keep
 *    the min(budget_m, F_h) best frames, ties to the lower frame index;
 *  - the kept frames and the current chunk are copied into out->k / out->v
 *    and the offsets written.
 * q, k_cache, v_cache: device tensors as above.  head_role, static_keep_mask:
 * host arrays as in fkv_plan.  workspace: device memory of at least the
 * bytes fkv_plan reports (NULL allowed when that figure is 0); its contents
 * on entry do not matter.  out->seg_score may be NULL. */
fkv_status_t fkv_compress(const fkv_desc_t *desc, const void *q, const void *k_cache,
                          const void *v_cache, const uint8_t *head_role,
                          const uint8_t *static_keep_mask, int32_t budget_m,
                          const fkv_ckv_t *out, void *workspace, size_t workspace_bytes,
                          void *stream);

/* fkv_compress followed by fkv_attend in one call ([S] 方法 › 输入与整体流程:
 * per layer, the cache is compressed and the current chunk attends over it):
 * the same compressed cache in *out and the same attention output in
 * attend_out [Nq, H, D] (element type of q), bit for bit, as those two calls
 * with the same attention workspace (attend_workspace / _bytes: optional, as
 * for fkv_attend).  A head's attention depends only on its own compressed
 * rows, so with bf16, when the attention runs one workgroup per (head,
 * 128-query tile), the heads without scored frames (static heads, dynamic
 * heads without history) start their attention on the library's side stream
 * as soon as their frames are copied, beside the scoring and selection of
 * the other heads, whose attention follows their copies on the given stream;
 * with a balanced attention schedule the two stages run one after the other.
 * The call is ordered on the given stream as a whole.  Arguments and errors
 * as for fkv_compress and fkv_attend; attend_out NULL is FKV_ERR_NULL. */
fkv_status_t fkv_compress_attend(const fkv_desc_t *desc, const void *q, const void *k_cache,
                                 const void *v_cache, const uint8_t *head_role,
                                 const uint8_t *static_keep_mask, int32_t budget_m,
                                 const fkv_ckv_t *out, void *workspace, size_t workspace_bytes,
                                 void *attend_out, void *attend_workspace,
                                 size_t attend_workspace_bytes, void *stream);

/* fkv_compress without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a fixed array of
 * FKV_SCRATCH_BYTES bytes inside the library, one copy per device, kept until
 * the process ends; the call itself allocates nothing.  A layer whose
 * workspace (fkv_plan's figure) exceeds FKV_SCRATCH_BYTES gets
 * FKV_ERR_WORKSPACE.  All calls on one device share that device's array:
 * calls that overlap on one device (other streams or threads) race, so order
 * them.  Otherwise the same arguments, results and errors as fkv_compress. */
#define FKV_SCRATCH_BYTES ((size_t)4 << 20)
fkv_status_t fkv_compress_noalloc(const fkv_desc_t *desc, const void *q, const void *k_cache,
                                  const void *v_cache, const uint8_t *head_role,
                                  const uint8_t *static_keep_mask, int32_t budget_m,
                                  const fkv_ckv_t *out, void *stream);

/* Measurement helper: fkv_compress with HIP events around its three stages;
 * waits for the device and writes the stage times in milliseconds to ms[3]
 * (scoring -- 0 when no head is scored --, selection, compaction). */
fkv_status_t fkv_compress_timed(const fkv_desc_t *desc, const void *q, const void *k_cache,
                                const void *v_cache, const uint8_t *head_role,
                                const uint8_t *static_keep_mask, int32_t budget_m,
                                const fkv_ckv_t *out, void *workspace, size_t workspace_bytes,
                                void *stream, float *ms);

/* ---- Rolling compressed cache (a chunk's compressed cache is the next
 * chunk's history) ----------------------------------------------------------
 * [S] 输出与工程收益: the compressed K/V replace the layer's cache.  Kept here
 * as the cache itself: after chunk c the compressed cache holds, per head, its
 * kept history frames and chunk c's (now finished) frames; frames not kept are
 * gone, and chunk c + 1 compresses that per-head history together with its own
 * current chunk.  The history of head h is then hist_frames[h] frames (of T
 * rows each) at rows [hist->tok_off[h], hist->tok_off[h+1]) of hist->k /
 * hist->v, which must agree with hist_frames[h] * T; desc->hist_frames is the
 * largest history any head may have (the row length of static_keep_mask). */

/* As fkv_plan, for per-head history lengths hist_frames[H] (host array,
 * 0 <= hist_frames[h] <= desc->hist_frames): a dynamic head keeps
 * min(m, hist_frames[h]) frames, a static head the frames its mask row marks,
 * which must all lie below hist_frames[h] (else FKV_ERR_SHAPE). */
fkv_status_t fkv_plan_ragged(const fkv_desc_t *desc, const int32_t *hist_frames,
                             const uint8_t *head_role, const uint8_t *static_keep_mask,
                             int32_t budget_m, int64_t *kept_tokens, size_t *workspace_bytes);

/* As fkv_compress, with each head's window = its history in `hist` (a
 * compressed cache written by an earlier fkv_compress or
 * fkv_compress_ragged; only k, v and tok_off are read) followed by the current
 * chunk cur_k / cur_v [F_c T, H, D] (token-major, device).  Scoring uses the
 * softmax over the head's whole window.  `out` receives the new compressed
 * cache and must not share buffers with `hist`. */
fkv_status_t fkv_compress_ragged(const fkv_desc_t *desc, const void *q, const fkv_ckv_t *hist,
                                 const int32_t *hist_frames, const void *cur_k,
                                 const void *cur_v, const uint8_t *head_role,
                                 const uint8_t *static_keep_mask, int32_t budget_m,
                                 const fkv_ckv_t *out, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Selection reused across the denoising steps of one chunk: copies the
 * current chunk cur_k / cur_v [F_c T, H, D] into the last F_c frames of every
 * head's range of ckv (which an earlier compression of this layer and chunk
 * wrote, offsets included); the kept history rows are left as they are. */
fkv_status_t fkv_refresh_current(const fkv_desc_t *desc, const void *cur_k, const void *cur_v,
                                 const fkv_ckv_t *ckv, void *stream);

/* Host helper: the keep mask of a static head's history in a rolling cache.
 * frame_ids[n_frames] are the absolute ids (>= 0, counting frames from the
 * start of the video; chunks are the aligned runs of cur_frames ids) of the
 * head's history frames, oldest first.  Marks the sink (id 0) and the first
 * and last frame of every chunk ([S] 关键模块 1 and 2: static heads attend to
 * chunk start and end positions), then, while more than cap are marked,
 * unmarks the oldest marked frame that is not a sink (sinks last).  With
 * cap = desc->hist_frames - cur_frames no history outgrows the window. */
fkv_status_t fkv_roll_static_mask(int32_t n_frames, const int32_t *frame_ids,
                                  int32_t cur_frames, int32_t cap, uint8_t *mask);

/* ---- FP8 compressed cache ([S] 行业影响 › 与现有产品/工作流的接口: the method
 * stacks with quantization) --------------------------------------------------
 * The cache rows are OCP FP8 e4m3 codes (1 byte per element, finite range
 * +-448, NaN 0x7F/0xFF): element x of head h is stored as the code of
 * x / scale[h] (an IEEE fp32 division, clamped to +-448, rounded to nearest
 * even).  Needs bf16 inputs with D = 128; ckv->k and ckv->v hold cap_tokens
 * rows of D bytes. */

/* As fkv_compress, writing an e4m3 cache.  kv_scales: host [2 H], the K
 * scales of heads 0 .. H-1, then the V scales (positive, finite). */
fkv_status_t fkv_compress_fp8(const fkv_desc_t *desc, const void *q, const void *k_cache,
                              const void *v_cache, const uint8_t *head_role,
                              const uint8_t *static_keep_mask, int32_t budget_m,
                              const float *kv_scales, const fkv_ckv_t *out, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Attention over an e4m3 cache on the fp8 matrix cores: the bf16 queries of
 * head h are quantized with scale[h] the same way, scores are
 * scale * (q_hat . k_hat) * q_scale * k_scale, outputs sum_j p_j v_hat_j *
 * v_scale / sum_j p_j with the weights p_j themselves rounded to e4m3 for
 * the value product (the sums use the same rounded weights).  scales: host
 * [3 H]: Q, K, V scales per head.  out as for fkv_attend (bf16).
 * workspace / workspace_bytes: optional, as for fkv_attend and of the same
 * size (fkv_attend_workspace of a bf16 descriptor): with it the launch takes
 * the same balanced schedules (pairs cut where that evens out the CUs, the
 * parts merged by a second kernel); NULL / 0: one workgroup per (head,
 * 128-query tile).  Calls that share a workspace must be ordered on one
 * stream.  The desc dtype must be FKV_BF16 (else FKV_ERR_DTYPE). */
fkv_status_t fkv_attend_fp8(const fkv_desc_t *desc, const void *q, const fkv_ckv_t *ckv,
                            const float *scales, void *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/* ---- Token-granular variant ----------------------------------------------
 * Static heads keep positions at token granularity ([S] 关键模块 1 and 2:
 * their attention sits on the start and end tokens of a chunk); dynamic heads
 * keep single tokens chosen by a participative score (Deep Forcing page,
 * 3.1: sink, recent and candidate zones, top-C candidates by the summed
 * query-key products of the recent queries).  History token t of a head is
 * window row t (frames oldest first); the plain-window layout of fkv_compress. */
typedef struct fkv_token_cfg {
  int32_t sink_frames;      /* leading history frames kept whole (every head)      */
  int32_t recent_frames;    /* trailing history frames kept whole (dynamic heads)  */
  int32_t budget_tokens;    /* C: candidate tokens a dynamic head keeps by score   */
  int32_t boundary_tokens;  /* L: tokens kept at each end of every history chunk
                               of cur_frames frames (static heads)                */
} fkv_token_cfg_t;

/* Kept rows and workspace bytes of fkv_compress_tokens (host only).  Static
 * head: its sink tokens plus the first and last L tokens of every aligned
 * history chunk (a trailing partial chunk included); dynamic head: sink and
 * recent frames plus min(C, candidates); every head then the current chunk. */
fkv_status_t fkv_plan_tokens(const fkv_desc_t *desc, const fkv_token_cfg_t *cfg,
                             const uint8_t *head_role, int64_t *kept_tokens,
                             size_t *workspace_bytes);

/* Token-granular compression of one layer.  Dynamic head h: candidate token j
 * (between the sink and recent zones) scores phi_j = sum_r q_r . k_j over the
 * sampled queries r = 0, s, 2s, ... of the current chunk; the C highest are
 * kept, ties to the lower token index.  Writes out->k, out->v (rows: kept
 * history tokens ascending, then the current chunk) and out->tok_off; row_src
 * (device [kept_tokens], may be NULL) receives the window token index of
 * every compacted row.  q, k_cache, v_cache, workspace as for fkv_compress. */
fkv_status_t fkv_compress_tokens(const fkv_desc_t *desc, const fkv_token_cfg_t *cfg,
                                 const void *q, const void *k_cache, const void *v_cache,
                                 const uint8_t *head_role, const fkv_ckv_t *out,
                                 int32_t *row_src, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* ---- Offline head profiling ([S] 关键模块 1) --------------------------------
 * Run on a few warm-up samples before inference; produces the head labels and
 * static keep masks that fkv_plan / fkv_compress take. */

/* Device workspace bytes fkv_profile_heads needs: H * n_s * (F_h + F_c) fp32,
 * n_s = ceil(Nq / query_stride). */
fkv_status_t fkv_profile_workspace(const fkv_desc_t *desc, size_t *workspace_bytes);

/* Attention mass by frame for every head: for each head h and window frame f,
 * the mean over the sampled queries (rows 0, s, 2s, ...; s = desc->query_stride,
 * 1 for all) of the softmax mass on frame f (softmax over the whole window,
 * scale * q.k logits), ADDED to mass_accum[h * (F_h + F_c) + f] (device fp32,
 * the caller zeroes it once and sums over samples / steps).  q, k_cache as for
 * fkv_compress (v is not needed). */
fkv_status_t fkv_profile_heads(const fkv_desc_t *desc, const void *q, const void *k_cache,
                               float *mass_accum, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Host: labels from the summed masses (host copy of mass_accum, n_calls
 * calls).  Chunk discontinuity of head h = mean mass of its boundary frames
 * (window frame f is one when f == 0 or f % F_c is 0 or F_c - 1: the sink and
 * the first and last frame of every aligned chunk) over the mean mass of the
 * others (NaN when there are no others or they get no mass).  The head is
 * static when discontinuity >= threshold (never for NaN), else dynamic; a
 * static head's mask row marks the history frames whose mean mass is at
 * least 1 / (F_h + F_c), a dynamic head's row is 0.  discontinuity[H] may be
 * NULL. */
fkv_status_t fkv_classify_heads(const fkv_desc_t *desc, const float *mass_sum, int32_t n_calls,
                                float threshold, uint8_t *head_role, uint8_t *static_keep_mask,
                                float *discontinuity);

/* Attention workspace.  The method's attention call takes only the queries
 * and the compressed cache; the (workspace, workspace_bytes) pair of
 * fkv_attend, fkv_attend_dense and fkv_attend_fp8 is an addition of this
 * library, optional (NULL, 0 is always accepted) and used only to balance
 * the work of a launch across the compute units.
 *
 * Bytes of the optional attention workspace for the current HIP device: with
 * it the bf16 attention (and the fp8 attention, which takes the same size)
 * balances its (head, 128-query) tiles over the resident workgroups (two per
 * compute unit): with at most one tile per compute unit it cuts tiles into a
 * main part and tails; with more tiles than resident workgroups it runs
 * whole tiles in rounds and halves those left for the last round so that it
 * is full.  The pieces of cut tiles are merged from partial results kept in
 * the workspace.  0 for fp32.  FKV_ERR_HIP when no device is visible. */
fkv_status_t fkv_attend_workspace(const fkv_desc_t *desc, size_t *workspace_bytes);

/* Attention of the whole query block over the compressed cache ([S]
 * 输出与工程收益): out[i, h] = sum_j softmax_j(scale * q[i,h].k_j) v_j over
 * head h's compressed rows, non-causal, fp32 accumulation, result rounded to
 * the element type.  ckv must hold what fkv_compress wrote (only k, v and
 * tok_off are read).  workspace: NULL (one workgroup per head and 128-query
 * tile) or device memory of at least fkv_attend_workspace's figure, else
 * FKV_ERR_WORKSPACE; its contents on entry do not matter, and calls that
 * share one workspace must be ordered (same stream). */
fkv_status_t fkv_attend(const fkv_desc_t *desc, const void *q, const fkv_ckv_t *ckv,
                        void *out, void *workspace, size_t workspace_bytes, void *stream);

/* Full-KV baseline ([S] 实验 › 实验设计: the method is measured against
 * keeping every history frame's KV): the same attention kernel over the whole
 * uncompressed window, every query seeing all N_win keys of its head.
 * q, k_cache, v_cache as for fkv_compress; out as for fkv_attend; workspace
 * as for fkv_attend (optional, an addition of this library). */
fkv_status_t fkv_attend_dense(const fkv_desc_t *desc, const void *q, const void *k_cache,
                              const void *v_cache, void *out, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Roofline calibration: the sustained bf16 MFMA rate of this device, from
 * chains of 32x32x16 MFMAs on register operands (two 4-wave workgroups per
 * CU, 8 * iters MFMAs per wave) on the default stream; waits for the device.
 * sink: any device buffer of 4 bytes (written only to keep the chains
 * alive, in practice never).  *tflops receives TFLOP/s. */
fkv_status_t fkv_mfma_peak(int32_t iters, float *sink, double *tflops);

/* Static text for a status code. */
const char *fkv_status_str(fkv_status_t status);

/* Detail of the last error on the calling thread ("" if none). */
const char *fkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FKV_H */
