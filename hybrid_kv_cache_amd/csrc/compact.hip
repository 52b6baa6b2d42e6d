// Gather / compaction of the kept frames into the ragged per-head cache.
// Forcing-KV summary page (ai-feeds.com, arXiv 2605.09681), 方法 ›
// 关键模块 › 2 (static positions are taken out by mask) and 输出与工程收益
// (the reduced K/V tensors replace the cache).  A pure copy: bytes in, the
// same bytes out.
//
// The selection kernel writes one CopySlot per (head, kept frame or current
// frame), in compacted order.  Workgroup b copies rows
// [64 c, 64 c + 64) of slot b / chunks (c = b % chunks) for K and V: every
// thread moves 16-byte pieces, each wave reads whole 256-byte head rows from
// the window (token-major, or a previous compressed cache for history
// frames) and writes them contiguously; eight loads are in flight per thread
// before the first store.  Loads and stores carry the non-temporal hint: the
// bytes are touched once, and the scoring running beside the copies keeps
// re-reading its K tiles from L2.  Without slots the kernel refreshes the
// current chunk of an existing compressed cache (selection reused across the
// denoising steps of one chunk).
//
// The copies that the plan fixes before any score is known (static heads'
// kept frames, every head's current chunk) have a kernel of their own, which
// runs beside the scoring; the selection then writes slots for the dynamic
// heads' kept history frames only.
#include "fkv_device.h"
#include "fkv_launch.h"

namespace fkv {
namespace {

__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  const int slot = blockIdx.x / a.chunks;
  const int c = blockIdx.x - slot * a.chunks;
  CopySlot sl;
  if (a.slots) {
    sl = a.slots[slot];
  } else {
    // current chunk only: frame j of head h goes to the last F_c frames of
    // the head's range
    sl.head = slot / a.F_c;
    const int j = slot - sl.head * a.F_c;
    sl.src_frame = a.fh[sl.head] + j;
    sl.dst_row = a.out_tok_off[sl.head + 1] - (int64_t)(a.F_c - j) * a.T;
  }
  copy_rows(a.win, a.fh[sl.head], sl, c, a.T, a.k_out, a.v_out);
}

// The compaction jobs fixed by the plan alone (static heads' kept frames,
// every head's current chunk): workgroup b copies chunk b % chunks of job
// b / chunks.  Independent of the scores, so it may run beside them.
__global__ __launch_bounds__(256) void compact_fixed_kernel(FixedCopyPlan p) {
  const int job = blockIdx.x / p.chunks;
  const int c = blockIdx.x - job * p.chunks;
  const CopySlot sl = fixed_slot(p, job);
  copy_rows(p.win, p.fh[sl.head], sl, c, p.T, p.k_out, p.v_out);
}

}  // namespace

hipError_t launch_compact_fixed(const FixedCopyPlan &p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.fixed_off_h[p.H] * p.chunks;
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(compact_fixed_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs &a, int total_slots, hipStream_t s) {
  if (total_slots <= 0) return hipSuccess;
  dim3 grid((unsigned)total_slots * (unsigned)a.chunks);
  hipLaunchKernelGGL(compact_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fkv
