// Kernel argument blocks and launchers of libfkv (host <-> device contract).
// Every launcher enqueues on the given stream and returns the launch status;
// none of them synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fkv {

constexpr int kMaxHeads = 64;
constexpr int kMaxHistFrames = 64;
constexpr int kMaxCurFrames = 8;

// Where the frames of each head's window live.  Frame f of head h is a
// history frame when f < fh[h] (fh: the head's history length, in the
// argument block that carries the view), else current-chunk frame f - fh[h].
//  - History, token-major window (hist_off null): row r of head h at
//    hist + r * tm_row_bytes + h * row_bytes.
//  - History, ragged per head (a previous compressed cache): row r of head h
//    at hist + (hist_off[h] + r) * row_bytes.
//  - Current chunk, token-major [F_c T, H, D]: row r of head h at
//    cur + r * tm_row_bytes + h * row_bytes.
struct WinView {
  const char *hist_k, *hist_v;
  const int64_t *hist_off;   // [H + 1] device row offsets, or null
  const char *cur_k, *cur_v;
  int64_t tm_row_bytes;      // H * D * elt
  int32_t row_bytes;         // D * elt
};

// One copy job of the compaction: the T rows of window frame src_frame of
// head `head` go to compacted rows dst_row .. dst_row + T - 1.
struct CopySlot {
  int32_t head;
  int32_t src_frame;
  int64_t dst_row;
};

// Per-(dynamic head, window frame, sampled query) log-sum-exp of the scaled
// logits in base 2: lse[(d * F_tot + f) * n_s + r] = log2 sum_{j in f} 2^(c q.k_j),
// with c = scale * log2(e), for f < fh[h] + F_c (F_tot: the largest window).
// Frame-major, so that the selection reads one frame of consecutive queries
// with coalesced loads.
struct ScoreArgs {
  const void *q;        // [Nq, H, D]
  WinView win;
  float *lse;           // [n_dyn, F_tot, n_s]
  int32_t H, D, T, F_c, F_tot, n_s, stride, n_dyn;
  int32_t n_qb;         // blocks of sampled queries per (head, frame) (set by the launcher)
  float c;
  int32_t dyn_heads[kMaxHeads];
  int32_t fh[kMaxHeads];
};

struct SelectArgs {
  const float *lse;     // [n_dyn, F_tot, n_s] (unused when n_dyn == 0)
  int32_t *seg_idx;     // [seg_off[H]]
  int32_t *seg_off;     // [H + 1]
  int64_t *tok_off;     // [H + 1]
  float *seg_score;     // [H * F_h] or null
  CopySlot *slots;      // [total_slots]
  int32_t H, T, F_h, F_c, F_tot, n_s, budget;  // F_h: row length of seg_score
  int32_t dyn_slots_only;  // 1: jobs only for dynamic heads' kept history frames
                           // (the others ran with the scoring), at slot_off_h
  int32_t fh[kMaxHeads];            // history frames of each head
  int32_t dyn_index[kMaxHeads];     // -1 static, else row block in lse
  uint64_t static_bits[kMaxHeads];  // kept history frames of static heads
  int32_t seg_off_h[kMaxHeads + 1];
  int32_t slot_off_h[kMaxHeads + 1];
  int64_t tok_off_h[kMaxHeads + 1];
};

// Head profiling: per (head, window frame) mean mass over the sampled
// queries, from the log-sum-exps of all heads (lse [H, F_tot, n_s]), added to
// out [H, F_tot].
struct ProfileArgs {
  const float *lse;
  float *out;
  int32_t H, F_tot, n_s;
};

// Token-granular compression (see tokens.hip).  History tokens of head h are
// t = 0 .. n_hist - 1 (frame-major), the current chunk n_hist .. n_hist + n_cur - 1;
// window row of token t, head h: (t * H + h) * D elements of q's element type.
struct TokenArgs {
  const void *q, *k, *v;    // [Nq, H, D], [N_win, H, D] x2
  char *k_out, *v_out;      // [rows, D]
  int32_t *src;             // [rows]: window token index of each compacted row
  int64_t *tok_off_out;     // [H + 1]: offsets written for attention
  float *qsum;              // [n_dyn, D]
  float *phi;               // [n_dyn, n_cand]
  int32_t H, D, elt, T, F_c, n_q, stride;
  int32_t n_hist, n_cur, sink_tok, recent_tok, cand_lo, cand_hi, n_cand, budget, boundary;
  int32_t n_dyn, max_rows;
  int32_t dyn_heads[kMaxHeads];
  int32_t dyn_index[kMaxHeads];   // -1: static
  int64_t tok_off_h[kMaxHeads + 1];
};

// Compaction.  With slots: one job per slot (head, window frame, rows).
// Without (slots null): the current chunk only, slot s = (head s / F_c,
// current frame s % F_c) going to the last F_c frames of the head's range in
// out_tok_off (the selection of an earlier call reused).
struct CompactArgs {
  const CopySlot *slots;
  WinView win;
  char *k_out;          // [rows, D]
  char *v_out;
  const int64_t *out_tok_off;  // [H + 1], read when slots is null
  int32_t T, F_c;
  int32_t chunks;         // ceil(T / kCompactRows)
  int32_t fh[kMaxHeads];
};
constexpr int kCompactRows = 64;

// The compaction jobs that do not depend on the scores (see fixed_slot in
// fkv_device.h): one workgroup per (job, kCompactRows-row chunk).
struct FixedCopyPlan {
  WinView win;
  char *k_out;          // [rows, D]
  char *v_out;
  int32_t H, T, chunks;           // chunks: ceil(T / kCompactRows)
  int32_t fh[kMaxHeads];
  int32_t fixed_off_h[kMaxHeads + 1];
  int32_t n_hist_fixed[kMaxHeads];
  int32_t kept[kMaxHeads];        // kept history frames of each head
  uint64_t static_bits[kMaxHeads];
  int64_t tok_off_h[kMaxHeads + 1];
};

struct AttendArgs {
  const void *q;          // [Nq, H, D]
  const void *k;          // ragged [rows, D] or window [N_win, H, D]
  const void *v;
  void *out;              // [Nq, H, D]
  const int64_t *tok_off; // ragged: [H + 1]; null for the dense window
  int64_t kv_row_stride;  // elements between consecutive keys of one head
  int32_t dense_len;      // window length when tok_off is null
  int32_t n_q, H, D;
  float c;                // scale * log2(e)
  float *part;            // partial-result slots (balanced schedules) or null
  int32_t n_wg;           // workgroups of the balanced schedules
  int32_t sched;          // 0: one workgroup per pair; 1: split; 2: rounds + halves
  int32_t slots_x;        // schedule 2: resident workgroups per XCD
  int32_t cut_max;        // schedule 2: most halved pairs on one XCD
  // Head subset (one workgroup per pair only): n_sel > 0 runs the heads
  // sel[0 .. n_sel) alone, with their row ranges [host_off[h], host_off[h+1])
  // of the ragged cache taken from these values instead of tok_off.
  int32_t n_sel;
  int32_t sel[kMaxHeads];
  int64_t host_off[kMaxHeads + 1];
};

hipError_t launch_score_bf16(const ScoreArgs &a, hipStream_t s);
hipError_t launch_score_f32(const ScoreArgs &a, hipStream_t s);
hipError_t launch_select(const SelectArgs &a, hipStream_t s);
hipError_t launch_profile(const ProfileArgs &a, hipStream_t s);
hipError_t launch_tokens(const TokenArgs &a, hipStream_t s);
hipError_t launch_compact(const CompactArgs &a, int total_slots, hipStream_t s);
hipError_t launch_compact_fixed(const FixedCopyPlan &p, hipStream_t s);
// Bytes of partial-result buffer that the balanced bf16 attention schedule
// needs on the current device (2 slots per workgroup, 2 workgroups per CU).
size_t attend_part_bytes();
// part / part_bytes: null / 0 for one workgroup per (head, query tile).
hipError_t launch_attend_bf16(const AttendArgs &a, void *part, size_t part_bytes, hipStream_t s);
// The schedule launch_attend_bf16 would pick (AttendArgs.sched) for a and the
// partial-result buffer.
int attend_bf16_schedule(const AttendArgs &a, void *part, size_t part_bytes);
// Fills the schedule fields of a (over all a.H heads, two workgroups per CU)
// for the partial-result buffer, null for one workgroup per pair; returns the
// combine kernel's workgroups (0: none).  launch_attend_combine merges the
// partial results of a launch planned so into a.out (bf16).
int plan_attend(AttendArgs &a, void *part, size_t part_bytes);
hipError_t launch_attend_combine(const AttendArgs &a, int blocks, hipStream_t s);
// The heads a.sel[0 .. a.n_sel) of the ragged cache, one workgroup per pair.
hipError_t launch_attend_bf16_heads(const AttendArgs &a, hipStream_t s);
hipError_t launch_attend_f32(const AttendArgs &a, hipStream_t s);

// Library-owned scratch array of fkv_compress_noalloc (scratch.hip): its size
// per device, and the device address of the current device's copy (looked up
// once per device; never the array's host-side name).
constexpr size_t kScratchBytes = (size_t)4 << 20;
hipError_t scratch_address(void **ptr);

}  // namespace fkv
