// Per-head frame selection and the ragged-layout bookkeeping.
//
// Forcing-KV summary page (ai-feeds.com, arXiv 2605.09681), 方法 › 关键模块:
//   2 (static structural pruning): a static head keeps a fixed, profiled set
//     of positions, taken by mask; here the mask is frame granular.
//   3 (dynamic similarity pruning): a dynamic head keeps the few frames with
//     the highest attention scores against the current queries.
// Score of history frame f of a dynamic head = mean over the sampled queries
// of the softmax mass of frame f (softmax over the head's whole window); the
// kept set is the min(m, fh) best of the head's fh history frames, ties
// broken by the lower frame index, emitted in ascending frame order.  (fh is
// F_h for every head of a plain window; a rolling cache gives each head its
// own history length.)
//
// One workgroup per head (16 waves; 4 when the window has more than 24
// frames).  Dynamic heads: one sampled query per
// thread at a time, the softmax over its frames in registers, masses summed
// per thread, then over each wave and over the waves in a fixed order
// (deterministic).
// Wave 0 then sorts the (score, frame) pairs with a 64-lane bitonic network
// (lane exchanges by DPP and permlane swaps, not the LDS crossbar) and marks
// the first m_eff.  Every head finally writes its seg_idx entries (bit rank =
// position), its offsets and its compaction slots.
#include "fkv_device.h"
#include "fkv_launch.h"

namespace fkv {
namespace {

// Sum over the 64 lanes of a wave, the total in every lane, without the
// LDS crossbar: DPP exchanges inside each row of 16 lanes (lane i with i ^ 1,
// i ^ 2, then the mirrored lane of its half row and of its row), then the
// row pairs (permlane16 swap) and the two halves (permlane32 swap).  The
// order of the additions is fixed, so the result is deterministic.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1, 0, 3, 2]: lane i ^ 1
  v += dpp<0x4E>(v);    // quad_perm [2, 3, 0, 1]: lane i ^ 2
  v += dpp<0x141>(v);   // row_half_mirror: the other quad of the half row
  v += dpp<0x140>(v);   // row_mirror: the other half row
  const LanePair r16 = permlane16_swap_copies(__builtin_bit_cast(uint32_t, v));
  v = __builtin_bit_cast(float, r16.a) + __builtin_bit_cast(float, r16.b);
  const LanePair r32 = permlane32_swap_copies(__builtin_bit_cast(uint32_t, v));
  return __builtin_bit_cast(float, r32.a) + __builtin_bit_cast(float, r32.b);
}

// The value of lane `lane ^ j` (j a power of two below 64; the loops that
// call it are unrolled, so j is a constant there): xor 1 and 2 by DPP quad
// permutes, xor 4 and 8 by DPP row shifts (lanes with the bit clear take the
// lane j above, the others the lane j below, always inside the row of 16),
// xor 16 and 32 by the permlane swaps of rows and halves.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int j, int lane) {
  const int x = (int)v;
  switch (j) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
    case 4: {
      const int up = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0xF, false);   // row_shl:4
      const int dn = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
      return (uint32_t)((lane & 4) ? dn : up);
    }
    case 8: {
      const int up = __builtin_amdgcn_update_dpp(0, x, 0x108, 0xF, 0xF, false);   // row_shl:8
      const int dn = __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
      return (uint32_t)((lane & 8) ? dn : up);
    }
    case 16: {
      const LanePair r = permlane16_swap_copies(v);   // rows [0,0,2,2] / [1,1,3,3]
      return (lane & 16) ? r.a : r.b;
    }
    default: {
      const LanePair r = permlane32_swap_copies(v);   // halves [lo,lo] / [hi,hi]
      return (lane & 32) ? r.a : r.b;
    }
  }
}

// (score, idx) a ranks before b: higher score first, then lower index.
__device__ __forceinline__ bool ranks_before(float sa, int ia, float sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

// Waves of the profiling workgroup, and of the selection workgroup when a
// head's window has more than 24 frames; up to 24 frames the selection uses
// 16 waves, so that one pass over the sampled queries covers up to 1024 of
// them (each pass waits for its loads once).
constexpr int kSelWaves = 4;
constexpr int kSelWavesWide = 16;

// Masses of one dynamic head: thread t takes sampled queries t, t + 64 W, ...;
// for each, the ft frame log-sum-exps (base 2; frame f at base[f * n_s + r],
// so that a wave reads each frame with one coalesced load) become a softmax
// over the head's window, whose first fh entries (the history) are added to
// per-thread sums.  The sums are reduced over each wave and stored per wave
// in part[w][f].
constexpr int kPartFrames = kMaxHistFrames + kMaxCurFrames;

template <int FT, int W>
__device__ __forceinline__ void accumulate_masses(const float *base, int n_s, int F_tot, int ft,
                                                  int fh, float (*part)[kPartFrames], int tid,
                                                  int lane, int wave) {
  float acc[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) acc[f] = 0.f;
  for (int r = tid; r < n_s; r += 64 * W) {
    float v[FT];
#pragma unroll
    for (int f = 0; f < FT; ++f) v[f] = f < ft ? base[(int64_t)f * n_s + r] : -INFINITY;
    float M = v[0];
#pragma unroll
    for (int f = 1; f < FT; ++f) M = fmaxf(M, v[f]);
    float S = 0.f;
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      v[f] = fast_exp2(v[f] - M);
      S += v[f];
    }
    const float inv = 1.f / S;
#pragma unroll
    for (int f = 0; f < FT; ++f) acc[f] += v[f] * inv;
  }
#pragma unroll
  for (int f = 0; f < FT && f < kPartFrames; ++f) {
    if (f < fh) {
      const float x = wave_sum(acc[f]);
      if (lane == 0) part[wave][f] = x;
    }
  }
}

template <int W>
__global__ __launch_bounds__(64 * W) void select_kernel(SelectArgs a) {
  __shared__ float part[W][kPartFrames];
  __shared__ unsigned long long kept_bits_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x;
  const int di = a.dyn_index[h];
  const int fh = a.fh[h];  // this head's history frames

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
    // One sampled query per thread: its frame values in registers, softmax
    // over frames, masses accumulated per thread; then a fixed-order
    // reduction over threads (deterministic).
    const float *base = a.lse + (int64_t)di * a.n_s * a.F_tot;
    const int ft = fh + a.F_c;
    if (W == kSelWavesWide)
      accumulate_masses<24, W>(base, a.n_s, a.F_tot, ft, fh, part, tid, lane, wave);
    else
      accumulate_masses<72, W>(base, a.n_s, a.F_tot, ft, fh, part, tid, lane, wave);
    __syncthreads();
    if (wave == 0) {
      float score = -INFINITY;
      if (lane < fh) {
        float sum = part[0][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += part[w][lane];
        score = sum / (float)a.n_s;
        if (a.seg_score) a.seg_score[(int64_t)h * a.F_h + lane] = score;
      } else if (a.seg_score && lane < a.F_h) {
        a.seg_score[(int64_t)h * a.F_h + lane] = __builtin_nanf("");
      }
      // Bitonic sort of 64 (score, frame) pairs into ranking order.  A NaN
      // score ranks like -inf, so the m_eff first entries are always real
      // frames (lanes >= fh carry -inf and larger indices).
      float s = score != score ? -INFINITY : score;
      int idx = lane;
#pragma unroll
      for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
          const float os = __builtin_bit_cast(float, lane_xor(__builtin_bit_cast(uint32_t, s), j, lane));
          const int oi = (int)lane_xor((uint32_t)idx, j, lane);
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
      const int m_eff = min(a.budget, fh);
      unsigned long long bits = lane < m_eff ? (1ull << idx) : 0ull;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const uint32_t lo = lane_xor((uint32_t)bits, off, lane);
        const uint32_t hi = lane_xor((uint32_t)(bits >> 32), off, lane);
        bits |= ((unsigned long long)hi << 32) | lo;
      }
      if (lane == 0) kept_bits_s = bits;
    }
  }
  __syncthreads();
  const unsigned long long bits = kept_bits_s;
  if (tid < fh && ((bits >> tid) & 1ull)) {
    const int pos = __popcll(bits & ((1ull << tid) - 1ull));
    a.seg_idx[a.seg_off_h[h] + pos] = tid;
  }
  // Compaction slots: kept history frames (ascending), then the current chunk
  // -- or, when the jobs that do not depend on the scores ran beside the
  // scoring, only a dynamic head's kept history frames.
  const int kept = __popcll(bits);
  const int nslots = !a.dyn_slots_only ? kept + a.F_c : (di >= 0 ? kept : 0);
  if (tid < nslots) {
    int src;
    if (tid < kept) {
      // tid-th set bit of `bits`
      unsigned long long b = bits;
      for (int i = 0; i < tid; ++i) b &= b - 1ull;
      src = __ffsll((long long)b) - 1;
    } else {
      src = fh + (tid - kept);
    }
    CopySlot sl;
    sl.head = h;
    sl.src_frame = src;
    sl.dst_row = a.tok_off_h[h] + (int64_t)tid * a.T;
    a.slots[a.slot_off_h[h] + tid] = sl;
  }
}

// Head profiling: the mean mass of every window frame of head blockIdx.x
// over the sampled queries, added to out[h * F_tot + f] (accumulates over
// calls; one workgroup per head, so the read-modify-write is unshared).
__global__ __launch_bounds__(64 * kSelWaves) void profile_kernel(ProfileArgs a) {
  __shared__ float part[kSelWaves][kPartFrames];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x;
  const float *base = a.lse + (int64_t)h * a.n_s * a.F_tot;
  if (a.F_tot <= 24)
    accumulate_masses<24, kSelWaves>(base, a.n_s, a.F_tot, a.F_tot, a.F_tot, part, tid, lane,
                                     wave);
  else
    accumulate_masses<72, kSelWaves>(base, a.n_s, a.F_tot, a.F_tot, a.F_tot, part, tid, lane,
                                     wave);
  __syncthreads();
  if (tid < a.F_tot) {
    float sum = part[0][tid];
#pragma unroll
    for (int w = 1; w < kSelWaves; ++w) sum += part[w][tid];
    a.out[(int64_t)h * a.F_tot + tid] += sum / (float)a.n_s;
  }
}

}  // namespace

hipError_t launch_profile(const ProfileArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(profile_kernel, dim3(a.H), dim3(64 * kSelWaves), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  if (a.F_tot <= 24)
    hipLaunchKernelGGL(select_kernel<kSelWavesWide>, dim3(a.H), dim3(64 * kSelWavesWide), 0, s, a);
  else
    hipLaunchKernelGGL(select_kernel<kSelWaves>, dim3(a.H), dim3(64 * kSelWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace fkv
