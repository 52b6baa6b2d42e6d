// Argument blocks and launchers of the FP8 (OCP e4m3) compressed cache:
// the quantizing compaction and the fp8 attention kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fkv_launch.h"

namespace fkv {

// Quantizing compaction: as CompactArgs (slots from the selection kernel),
// writing code(row_value / scale[h]) as e4m3 bytes, rows of D bytes.
struct CompactFp8Args {
  const CopySlot *slots;
  WinView win;              // bf16 window
  uint8_t *k_out, *v_out;   // [rows, D]
  int32_t T, chunks, D;
  int32_t fh[kMaxHeads];
  float k_scale[kMaxHeads];
  float v_scale[kMaxHeads];
};

// Per-head e4m3 scales of K and V and the head dimension, for the
// quantizing copies of the fixed compaction jobs.
struct Fp8Scales {
  int32_t D;
  float k_scale[kMaxHeads];
  float v_scale[kMaxHeads];
};

// fp8 attention over an e4m3 compressed cache (D = 128).  Queries are bf16
// and quantized per head in the kernel (q / q_scale[h]); scores are
// (q_hat . k_hat) q_scale k_scale, values v_hat v_scale.
struct AttendFp8Args {
  const void *q;            // [Nq, H, 128] bf16
  const uint8_t *k, *v;     // [rows, 128] e4m3
  void *out;                // [Nq, H, 128] bf16
  const int64_t *tok_off;   // [H + 1]
  int32_t n_q, H;
  float c;                  // softmax scale * log2(e)
  float q_scale[kMaxHeads];
  float k_scale[kMaxHeads];
  float v_scale[kMaxHeads];
  // Schedule (set by launch_attend_fp8, as for the bf16 kernel).
  float *part;              // partial-result slots or null
  int32_t n_wg, sched, slots_x, cut_max;
};

hipError_t launch_compact_fp8(const CompactFp8Args &a, int total_slots, hipStream_t s);
// The quantizing copies of the fixed compaction jobs of p.
hipError_t launch_compact_fp8_fixed(const FixedCopyPlan &p, const Fp8Scales &sc, hipStream_t s);
// part / part_bytes: the bf16 attention's partial-result buffer
// (attend_part_bytes()) for its balanced schedules, or null / 0 for one
// workgroup per (head, query tile) pair.
hipError_t launch_attend_fp8(const AttendFp8Args &a, void *part, size_t part_bytes, hipStream_t s);

}  // namespace fkv
