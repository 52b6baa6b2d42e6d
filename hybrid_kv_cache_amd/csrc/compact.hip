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
// before the first store.  Without slots the kernel refreshes the current
// chunk of an existing compressed cache (selection reused across the
// denoising steps of one chunk).
#include "fkv_device.h"
#include "fkv_launch.h"

namespace fkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs a) {
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
  const int r0 = c * kCompactRows;
  const int nrows = min(kCompactRows, a.T - r0);
  const int row_bytes = a.win.row_bytes;
  const int v16 = row_bytes >> 4;          // 16-byte pieces per row
  const int items = nrows * v16;
  int64_t src_stride;
  const char *ks = frame_rows(a.win, false, sl.head, a.fh[sl.head], sl.src_frame, a.T,
                              &src_stride) + r0 * src_stride;
  const char *vs = frame_rows(a.win, true, sl.head, a.fh[sl.head], sl.src_frame, a.T,
                              &src_stride) + r0 * src_stride;
  char *kd = a.k_out + (sl.dst_row + r0) * row_bytes;
  char *vd = a.v_out + (sl.dst_row + r0) * row_bytes;

  constexpr int U = 4;
  for (int base = 0; base < items; base += kThreads * U) {
    u32x4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * kThreads + threadIdx.x;
      if (idx < items) {
        const int r = idx / v16, p = idx - r * v16;
        const int64_t so = r * src_stride + p * 16;
        kr[u] = ld16(ks + so);
        vr[u] = ld16(vs + so);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * kThreads + threadIdx.x;
      if (idx < items) {
        st16(kd + (int64_t)idx * 16, kr[u]);
        st16(vd + (int64_t)idx * 16, vr[u]);
      }
    }
  }
}

}  // namespace

hipError_t launch_compact(const CompactArgs &a, int total_slots, hipStream_t s) {
  if (total_slots <= 0) return hipSuccess;
  dim3 grid((unsigned)total_slots * (unsigned)a.chunks);
  hipLaunchKernelGGL(compact_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fkv
