// Per-head frame selection and the ragged-layout bookkeeping.
//
// Forcing-KV summary page (ai-feeds.com, arXiv 2605.09681), 方法 › 关键模块:
//   2 (static structural pruning): a static head keeps a fixed, profiled set
//     of positions, taken by mask; here the mask is frame granular.
//   3 (dynamic similarity pruning): a dynamic head keeps the few frames with
//     the highest attention scores against the current queries.
// Score of history frame f of a dynamic head = mean over the sampled queries
// of the softmax mass of frame f (softmax over the whole window); the kept
// set is the min(m, F_h) best frames, ties broken by the lower frame index,
// emitted in ascending frame order.
//
// One workgroup (16 waves) per head.  Dynamic heads: each wave walks every
// 16th sampled query, lane f holding frame f's log-sum-exp; wave-wide
// max / sum give that query's per-frame masses, accumulated per lane; the
// 16 partial sums are added in a fixed order (deterministic).
// Wave 0 then sorts the (score, frame) pairs with a 64-lane bitonic network
// and marks the first m_eff.  Every head finally writes its seg_idx entries
// (bit rank = position), its offsets and its compaction slots.
#include "fkv_device.h"
#include "fkv_launch.h"

namespace fkv {
namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// (score, idx) a ranks before b: higher score first, then lower index.
__device__ __forceinline__ bool ranks_before(float sa, int ia, float sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

constexpr int kSelWaves = 16;

__global__ __launch_bounds__(64 * kSelWaves) void select_kernel(SelectArgs a) {
  __shared__ float part[kSelWaves][128];
  __shared__ unsigned long long kept_bits_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x;
  const int di = a.dyn_index[h];

  if (tid == 0) {
    a.seg_off[h] = a.seg_off_h[h];
    a.tok_off[h] = a.tok_off_h[h];
    if (h == a.H - 1) {
      a.seg_off[a.H] = a.seg_off_h[a.H];
      a.tok_off[a.H] = a.tok_off_h[a.H];
    }
  }

  if (di < 0) {
    if (tid == 0) kept_bits_s = a.static_bits[h];
    if (a.seg_score && tid < a.F_h) a.seg_score[(int64_t)h * a.F_h + tid] = __builtin_nanf("");
  } else {
    // Per-lane accumulation of masses over this wave's sampled queries, four
    // rows per batch with their loads issued together.
    float acc0 = 0.f, acc1 = 0.f;
    const bool two = a.F_tot > 64;
    const float *base = a.lse + (int64_t)di * a.n_s * a.F_tot;
    for (int r0 = wave; r0 < a.n_s; r0 += 4 * kSelWaves) {
      float v0[4], v1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u * kSelWaves;
        const bool in = r < a.n_s;
        const float *row = base + (int64_t)(in ? r : 0) * a.F_tot;
        v0[u] = (in && lane < a.F_tot) ? row[lane] : -INFINITY;
        v1[u] = (in && two && lane + 64 < a.F_tot) ? row[lane + 64] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (r0 + u * kSelWaves >= a.n_s) break;
        const float M = wave_max(fmaxf(v0[u], v1[u]));
        const float e0 = fast_exp2(v0[u] - M), e1 = fast_exp2(v1[u] - M);
        const float inv = 1.f / wave_sum(e0 + e1);
        acc0 += e0 * inv;
        acc1 += e1 * inv;
      }
    }
    part[wave][lane] = acc0;
    part[wave][lane + 64] = acc1;
    __syncthreads();
    if (wave == 0) {
      float score = -INFINITY;
      if (lane < a.F_h) {
        float sum = part[0][lane];
#pragma unroll
        for (int w = 1; w < kSelWaves; ++w) sum += part[w][lane];
        score = sum / (float)a.n_s;
        if (a.seg_score) a.seg_score[(int64_t)h * a.F_h + lane] = score;
      }
      // Bitonic sort of 64 (score, frame) pairs into ranking order.  A NaN
      // score ranks like -inf, so the m_eff first entries are always real
      // frames (lanes >= F_h carry -inf and larger indices).
      float s = score != score ? -INFINITY : score;
      int idx = lane;
#pragma unroll
      for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
          const float os = __shfl_xor(s, j, 64);
          const int oi = __shfl_xor(idx, j, 64);
          const bool lower = (lane & j) == 0;
          const bool ascending = (lane & k) == 0;
          const bool other_first = ranks_before(os, oi, s, idx);
          // The lower lane of an ascending pair keeps the element that ranks
          // first; descending pairs the reverse.
          const bool take = (lower == ascending) ? other_first : !other_first;
          if (take) {
            s = os;
            idx = oi;
          }
        }
      }
      // Lane i now holds the i-th ranked frame; OR together the first m_eff.
      unsigned long long bits = lane < a.m_eff ? (1ull << idx) : 0ull;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) bits |= __shfl_xor(bits, off, 64);
      if (lane == 0) kept_bits_s = bits;
    }
  }
  __syncthreads();
  const unsigned long long bits = kept_bits_s;
  if (tid < a.F_h && ((bits >> tid) & 1ull)) {
    const int pos = __popcll(bits & ((1ull << tid) - 1ull));
    a.seg_idx[a.seg_off_h[h] + pos] = tid;
  }
  // Compaction slots: kept history frames (ascending), then the current chunk.
  const int kept = __popcll(bits);
  const int nslots = kept + a.F_c;
  if (tid < nslots) {
    int src;
    if (tid < kept) {
      // tid-th set bit of `bits`
      unsigned long long b = bits;
      for (int i = 0; i < tid; ++i) b &= b - 1ull;
      src = __ffsll((long long)b) - 1;
    } else {
      src = a.F_h + (tid - kept);
    }
    CopySlot sl;
    sl.head = h;
    sl.src_frame = src;
    sl.dst_row = a.tok_off_h[h] + (int64_t)tid * a.T;
    a.slots[a.slot_off_h[h] + tid] = sl;
  }
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(a.H), dim3(64 * kSelWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace fkv
