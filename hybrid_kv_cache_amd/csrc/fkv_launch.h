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

// One copy job of the compaction: the T rows of window frame src_frame of
// head `head` go to compacted rows dst_row .. dst_row + T - 1.
struct CopySlot {
  int32_t head;
  int32_t src_frame;
  int64_t dst_row;
};

// Per-(dynamic head, sampled query, window frame) log-sum-exp of the scaled
// logits in base 2: lse[(d * n_s + r) * F_tot + f] = log2 sum_{j in f} 2^(c q.k_j),
// with c = scale * log2(e).
struct ScoreArgs {
  const void *q;        // [Nq, H, D]
  const void *k;        // [N_win, H, D]
  float *lse;           // [n_dyn, n_s, F_tot]
  int32_t H, D, T, F_tot, n_s, stride, n_dyn;
  float c;
  int32_t dyn_heads[kMaxHeads];
};

struct SelectArgs {
  const float *lse;     // [n_dyn, n_s, F_tot] (unused when n_dyn == 0)
  int32_t *seg_idx;     // [seg_off[H]]
  int32_t *seg_off;     // [H + 1]
  int64_t *tok_off;     // [H + 1]
  float *seg_score;     // [H * F_h] or null
  CopySlot *slots;      // [total_slots]
  int32_t H, T, F_h, F_c, F_tot, n_s, m_eff;
  int32_t dyn_index[kMaxHeads];     // -1 static, else row block in lse
  uint64_t static_bits[kMaxHeads];  // kept history frames of static heads
  int32_t seg_off_h[kMaxHeads + 1];
  int32_t slot_off_h[kMaxHeads + 1];
  int64_t tok_off_h[kMaxHeads + 1];
};

struct CompactArgs {
  const CopySlot *slots;
  const char *k;        // [N_win, H, D] bytes
  const char *v;
  char *k_out;          // [rows, D]
  char *v_out;
  int64_t src_row_bytes;  // H * D * elt
  int32_t row_bytes;      // D * elt
  int32_t head_bytes;     // D * elt (offset of head h inside a token row = h * head_bytes)
  int32_t T;
  int32_t chunks;         // ceil(T / kCompactRows)
};
constexpr int kCompactRows = 64;

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
  float *part;            // partial-result slots (balanced bf16 schedule) or null
  int32_t n_wg;           // workgroups of the balanced schedule
};

hipError_t launch_score_bf16(const ScoreArgs &a, hipStream_t s);
hipError_t launch_score_f32(const ScoreArgs &a, hipStream_t s);
hipError_t launch_select(const SelectArgs &a, hipStream_t s);
hipError_t launch_compact(const CompactArgs &a, int total_slots, hipStream_t s);
// Bytes of partial-result buffer that the balanced bf16 attention schedule
// needs on the current device (2 slots per workgroup, 2 workgroups per CU).
size_t attend_part_bytes();
// part / part_bytes: null / 0 for one workgroup per (head, query tile).
hipError_t launch_attend_bf16(const AttendArgs &a, void *part, size_t part_bytes, hipStream_t s);
hipError_t launch_attend_f32(const AttendArgs &a, hipStream_t s);

}  // namespace fkv
