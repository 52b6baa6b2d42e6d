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
// Wave 0 then ranks the frames (lane f counts the frames whose (score,
// index) pair ranks before its own, reading them by readlane) and keeps those
// of rank below m_eff, a ballot giving the kept-frame bit mask.  Every head
// finally writes its seg_idx entries (bit rank = position), its offsets and
// its compaction slots.
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
__device__ __forceinline__ void accumulate_masses(const float *base, int n_s, int ft, int fh,
                                                  float (*part)[kPartFrames], int tid,
                                                  int lane, int wave) {
  if (wave * 64 >= n_s) {
    // No sampled query reaches this wave: its partial sums are 0.
    if (lane < fh && lane < kPartFrames) part[wave][lane] = 0.f;
    return;
  }
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
      accumulate_masses<24, W>(base, a.n_s, ft, fh, part, tid, lane, wave);
    else
      accumulate_masses<72, W>(base, a.n_s, ft, fh, part, tid, lane, wave);
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
      // Rank of frame `lane` among the head's fh history frames: the number
      // of frames that rank before it (higher score, ties to the lower
      // index; a NaN score ranks like -inf).  The ranks are a permutation
      // of 0 .. fh - 1, and the frames of rank below m_eff are kept: the
      // first m_eff of the ranking order, as a bit mask by frame index.
      const float s = score != score ? -INFINITY : score;
      int rank = 0;
      for (int g = 0; g < fh; ++g) {
        const float sg = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), g));
        rank += ranks_before(sg, g, s, lane) ? 1 : 0;
      }
      const int m_eff = min(a.budget, fh);
      const unsigned long long bits = __ballot(lane < fh && rank < m_eff);
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
    accumulate_masses<24, kSelWaves>(base, a.n_s, a.F_tot, a.F_tot, part, tid, lane, wave);
  else
    accumulate_masses<72, kSelWaves>(base, a.n_s, a.F_tot, a.F_tot, part, tid, lane, wave);
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
