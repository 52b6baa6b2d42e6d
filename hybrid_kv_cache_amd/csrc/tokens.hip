// Token-granular compression: a static head keeps its sink frames and the
// tokens at both ends of every history chunk; a dynamic head keeps sink and
// recent frames whole and the top C candidate tokens between them by their
// participative score phi_j = sum_r q_r . k_j over the sampled current-chunk
// queries.  Forcing-KV summary page (ai-feeds.com, arXiv 2605.09681),
// 方法 › 关键模块 1 and 2 (static heads: start and end tokens of a chunk);
// Deep Forcing page, 3.1 动态token筛选算法 (sink / recent / candidate zones,
// top-C by summed query-key products).
//
// Kernels, in launch order:
//   qsum_kernel    per dynamic head, Qsum[d] = sum over sampled rows of q[r, h, d]
//                  (fp32, fixed grouping of the rows);
//   phi_kernel     phi[j] = k_j . Qsum for every candidate token (one thread
//                  per token, fp32, dims in order) -- sum_r q_r . k_j regrouped;
//   token_select_kernel
//                  one workgroup per head: the kept history tokens in
//                  ascending order (static: pattern flags; dynamic: a 4-pass
//                  8-bit radix select finds the C-th largest phi, ties to the
//                  lower index; each thread then walks its own run of
//                  candidates, placed by one scan of the per-thread counts),
//                  written as the window token index of every compacted row,
//                  plus the current chunk;
//   gather_kernel  copies the K and V rows those indices name.
#include "fkv_device.h"
#include "fkv_launch.h"

namespace fkv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kLdsKeys = 24576;   // candidates staged in LDS (96 KiB)
constexpr int kMaxPer = kLdsKeys / kSelThreads;  // candidates per thread when staged

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }

// 1024 threads per dynamic head.  Each sampled row is read as 16-byte
// pieces: tpr = D / vec threads per row (vec elements each), R = 1024 / tpr
// row groups; group g takes the sampled rows g, g + R, g + 2R, ... (four
// rows in flight, added in row order).  The groups' partial sums are then
// added per dimension in group order.
template <typename T>
__global__ __launch_bounds__(kSelThreads) void qsum_kernel(TokenArgs a) {
  constexpr int vec = 16 / sizeof(T);
  __shared__ float part[kSelThreads * vec];   // [R][D]
  const int di = blockIdx.x, h = a.dyn_heads[di];
  const int tid = threadIdx.x, D = a.D;
  const int tpr = D / vec, R = kSelThreads / tpr;
  const int c = tid % tpr, g = tid / tpr;
  const int64_t hd = (int64_t)a.H * D;
  const int n_s = (a.n_q + a.stride - 1) / a.stride;
  const int64_t step = (int64_t)R * a.stride * hd;
  const T *p = reinterpret_cast<const T *>(a.q) + (int64_t)g * a.stride * hd + (int64_t)h * D +
               c * vec;
  float s[vec];
#pragma unroll
  for (int e = 0; e < vec; ++e) s[e] = 0.f;
  auto add = [&](const u32x4 &x) {
    const T *v = reinterpret_cast<const T *>(&x);
#pragma unroll
    for (int e = 0; e < vec; ++e) s[e] += to_f32<T>(v[e]);
  };
  int j = g;
  for (; j + 3 * R < n_s; j += 4 * R, p += 4 * step) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const u32x4 *>(p + u * step);
#pragma unroll
    for (int u = 0; u < 4; ++u) add(x[u]);
  }
  for (; j < n_s; j += R, p += step) add(*reinterpret_cast<const u32x4 *>(p));
#pragma unroll
  for (int e = 0; e < vec; ++e) part[g * D + c * vec + e] = s[e];
  __syncthreads();
  if (tid < D) {
    float t = part[tid];
    for (int k = 1; k < R; ++k) t += part[k * D + tid];
    a.qsum[di * D + tid] = t;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void phi_kernel(TokenArgs a) {
  __shared__ float qs[128];
  const int di = blockIdx.y, h = a.dyn_heads[di];
  for (int d = threadIdx.x; d < a.D; d += 256) qs[d] = a.qsum[di * a.D + d];
  __syncthreads();
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.n_cand) return;
  const int64_t tok = a.cand_lo + j;
  const T *k = reinterpret_cast<const T *>(a.k) + (tok * a.H + h) * a.D;
  float s = 0.f;
  for (int d = 0; d < a.D; d += 8) {
    T x[8];
    *reinterpret_cast<u32x4 *>(x) = *reinterpret_cast<const u32x4 *>(k + d);
    if constexpr (sizeof(T) == 4) {
      *reinterpret_cast<u32x4 *>(x + 4) = *reinterpret_cast<const u32x4 *>(k + d + 4);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(to_f32<T>(x[e]), qs[d + e], s);
  }
  a.phi[(int64_t)di * a.n_cand + j] = s;
}

// Order-preserving map of a float to an unsigned key (larger float, larger key).
__device__ __forceinline__ uint32_t sort_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the workgroup (1024 threads, 16 waves) in
// thread order; *total gets the sum.  Uses wsum[16] in LDS.
__device__ __forceinline__ int block_excl_scan(int v, int *wsum, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const int t = wsum[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Static pattern over a run of history tokens [lo, hi): calls f(t) for each
// kept token in order (sink tokens, and the first and last `boundary` tokens
// of every aligned chunk of F_c frames).  One division per run.
template <typename F>
__device__ __forceinline__ void static_run(const TokenArgs &a, int lo, int hi, F f) {
  const int chunk = a.F_c * a.T;
  int c0 = (lo / chunk) * chunk;
  for (int t = lo; t < hi; ++t) {
    if (t >= c0 + chunk) c0 += chunk;
    const int c1 = min(c0 + chunk, a.n_hist);
    if (t < a.sink_tok || t - c0 < a.boundary || c1 - t <= a.boundary) f(t);
  }
}

// Wave 0 finds the digit of the next radix pass: the largest d such that the
// bins above d hold fewer than `need` keys (bins from 255 down, four per lane).
__device__ __forceinline__ void pick_digit(const int *hist, uint32_t prefix, int shift, int need,
                                           uint32_t *s_prefix, int *s_remaining) {
  const int lane = threadIdx.x & 63;
  int c[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = hist[255 - 4 * lane - i];
    sum += c[i];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  int acc = incl - sum;  // keys in the bins above this lane's four
  int hit = -1, before = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (hit < 0 && acc + c[i] >= need) {
      hit = 255 - 4 * lane - i;
      before = acc;
    }
    acc += c[i];
  }
  const unsigned long long hits = __ballot(hit >= 0);
  if (hits != 0 && lane == __ffsll((long long)hits) - 1) {
    *s_prefix = prefix | ((uint32_t)hit << shift);
    *s_remaining = need - before;
  }
}

// Adds 1 to hist[bin] for every lane with take set, one LDS atomic per
// distinct bin of the wave: the first remaining lane's bin leads, the lanes
// with the same bin are counted by a ballot.  For the first radix pass, where
// the keys of a wave share a few bins (sign and top exponent bits), this
// replaces a many-way serialised atomic per lane (-10% on the whole token
// compression at 480P); on the later passes, whose bins are spread, the
// plain per-lane atomics are faster.
__device__ __forceinline__ void wave_hist_add(int *hist, uint32_t bin, bool take) {
  unsigned long long todo = __ballot(take);
  const int lane = threadIdx.x & 63;
  while (todo) {
    const int leader = __ffsll((long long)todo) - 1;
    const uint32_t lbin = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
    const unsigned long long same = __ballot(take && bin == lbin) & todo;
    if (lane == leader) atomicAdd(&hist[lbin], __popcll(same));
    todo &= ~same;
  }
}

__global__ __launch_bounds__(kSelThreads) void token_select_kernel(TokenArgs a) {
  constexpr int kWaves = kSelThreads / 64;
  __shared__ uint32_t lds_keys[kLdsKeys];
  __shared__ int whist[kWaves * 256];
  __shared__ int hist[256];
  __shared__ int wsum[kSelThreads / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  const int h = blockIdx.x, tid = threadIdx.x;
  const int di = a.dyn_index[h];
  int32_t *out = a.src + a.tok_off_h[h];
  if (tid == 0) {
    a.tok_off_out[h] = a.tok_off_h[h];
    if (h == a.H - 1) a.tok_off_out[a.H] = a.tok_off_h[a.H];
  }
  int pos = 0;  // rows written so far (uniform)

  if (di < 0) {
    // static pattern over the history: thread t walks its own run of tokens,
    // one scan of the per-thread counts places them in token order
    const int per = (a.n_hist + kSelThreads - 1) / kSelThreads;
    const int lo = min(tid * per, a.n_hist), hi = min(lo + per, a.n_hist);
    int cnt = 0;
    static_run(a, lo, hi, [&](int) { ++cnt; });
    int total;
    int p = block_excl_scan(cnt, wsum, &total);
    static_run(a, lo, hi, [&](int t) { out[p++] = t; });
    pos = total;
  } else {
    // sink zone
    for (int t = tid; t < a.sink_tok; t += kSelThreads) out[t] = t;
    pos = a.sink_tok;
    const float *phi = a.phi + (int64_t)di * a.n_cand;
    const int n = a.n_cand, c = min(a.budget, n);
    // The keys are read 6 times; up to kLdsKeys of them are staged in LDS.
    const bool in_lds = n <= kLdsKeys;
    if (in_lds) {
      for (int j = tid; j < n; j += kSelThreads) lds_keys[j] = sort_key(phi[j]);
      __syncthreads();
    }
    auto key_at = [&](int j) -> uint32_t { return in_lds ? lds_keys[j] : sort_key(phi[j]); };
    uint32_t thr = 0;
    int remaining = 0;  // keys equal to thr to take, lowest index first
    if (c > 0 && c < n) {
      // radix select of the c-th largest key, 8 bits per pass from the top
      uint32_t prefix = 0;
      int need = c;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        // one histogram per wave (keys of similar size share their top bits,
        // so a single one would serialise every wave on a few bins)
        for (int i = tid; i < kWaves * 256; i += kSelThreads) whist[i] = 0;
        __syncthreads();
        int *mine = whist + (tid >> 6) * 256;
        const uint32_t want = prefix >> (shift + 8);
        int j = tid;
        if (pass == 0) {
          // wave-aggregated adds: the keys of a wave crowd into few bins
          for (; j - tid < n; j += kSelThreads) {
            const bool in = j < n;
            const uint32_t key = in ? key_at(j) : 0u;
            wave_hist_add(mine, (key >> shift) & 255u,
                          in && (pass == 0 || (key >> (shift + 8)) == want));
          }
        } else {
          for (; j + 3 * kSelThreads < n; j += 4 * kSelThreads) {
            uint32_t k4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) k4[u] = key_at(j + u * kSelThreads);
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if ((k4[u] >> (shift + 8)) == want) atomicAdd(&mine[(k4[u] >> shift) & 255u], 1);
          }
          for (; j < n; j += kSelThreads) {
            const uint32_t key = key_at(j);
            if ((key >> (shift + 8)) == want) atomicAdd(&mine[(key >> shift) & 255u], 1);
          }
        }
        __syncthreads();
        if (tid < 256) {
          int sum = 0;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) sum += whist[w * 256 + tid];
          hist[tid] = sum;
        }
        __syncthreads();
        if (tid < 64) pick_digit(hist, prefix, shift, need, &s_prefix, &s_remaining);
        __syncthreads();
        prefix = s_prefix;
        need = s_remaining;
        __syncthreads();
      }
      thr = prefix;
      remaining = need;
    }
    // Kept candidates in index order: key > thr, or key == thr among the
    // first `remaining` such (all when c == n, none when c == 0).  Thread t
    // walks its own run; with gt / eq counts before a candidate, its row is
    // gt_before + min(eq_before, remaining).
    const int per = (n + kSelThreads - 1) / kSelThreads;
    const int lo = min(tid * per, n), hi = min(lo + per, n);
    const bool all = c >= n, none = c == 0;
    int gt = 0, eq = 0;
    if (!all && !none) {
      for (int j = lo; j < hi; ++j) {
        const uint32_t key = key_at(j);
        gt += key > thr;
        eq += key == thr;
      }
    }
    int gt_total, eq_total;
    int gt_b = block_excl_scan(gt, wsum, &gt_total);
    int eq_b = block_excl_scan(eq, wsum, &eq_total);
    if (all) {
      for (int j = tid; j < n; j += kSelThreads) out[pos + j] = a.cand_lo + j;
    } else if (!none && in_lds) {
      // This thread's keys into registers, then the key array becomes the
      // staging of the kept indices in row order, copied out coalesced.
      uint32_t kr[kMaxPer];
#pragma unroll
      for (int i = 0; i < kMaxPer; ++i) kr[i] = lo + i < hi ? lds_keys[lo + i] : 0u;
      __syncthreads();
      int32_t *stage = reinterpret_cast<int32_t *>(lds_keys);
#pragma unroll
      for (int i = 0; i < kMaxPer; ++i) {
        if (lo + i < hi) {
          const int row = gt_b + min(eq_b, remaining);
          if (kr[i] > thr) {
            stage[row] = a.cand_lo + lo + i;
            ++gt_b;
          } else if (kr[i] == thr) {
            if (eq_b < remaining) stage[row] = a.cand_lo + lo + i;
            ++eq_b;
          }
        }
      }
      __syncthreads();
      for (int r = tid; r < c; r += kSelThreads) out[pos + r] = stage[r];
    } else if (!none) {
      for (int j = lo; j < hi; ++j) {
        const uint32_t key = key_at(j);
        const int row = gt_b + min(eq_b, remaining);
        if (key > thr) {
          out[pos + row] = a.cand_lo + j;
          ++gt_b;
        } else if (key == thr) {
          if (eq_b < remaining) out[pos + row] = a.cand_lo + j;
          ++eq_b;
        }
      }
    }
    pos += c;
    // recent zone
    for (int t = tid; t < a.recent_tok; t += kSelThreads) out[pos + t] = a.cand_hi + t;
    pos += a.recent_tok;
  }
  // current chunk
  for (int t = tid; t < a.n_cur; t += kSelThreads) out[pos + t] = a.n_hist + t;
}

// Rows [64 b, 64 b + 64) of head blockIdx.y's compacted range: K and V rows of
// the window tokens src names, 16 bytes per thread and step.
__global__ __launch_bounds__(256) void gather_kernel(TokenArgs a) {
  const int h = blockIdx.y;
  const int64_t lo = a.tok_off_h[h], n = a.tok_off_h[h + 1] - lo;
  const int r0 = blockIdx.x * 64;
  if (r0 >= n) return;
  const int rows = (int)min((int64_t)64, n - r0);
  const int row_bytes = a.D * a.elt;
  const int v16 = row_bytes >> 4;                 // a power of two (D 64 or 128)
  const int v16_shift = __builtin_ctz((unsigned)v16);
  const int64_t tm = (int64_t)a.H * row_bytes;
  const char *kb = reinterpret_cast<const char *>(a.k) + (int64_t)h * row_bytes;
  const char *vb = reinterpret_cast<const char *>(a.v) + (int64_t)h * row_bytes;
  for (int i = threadIdx.x; i < rows * v16; i += 256) {
    const int r = i >> v16_shift, p = i & (v16 - 1);
    const int64_t t = a.src[lo + r0 + r];
    const int64_t so = t * tm + p * 16;
    const int64_t d = (lo + r0 + r) * row_bytes + p * 16;
    st16(a.k_out + d, ld16(kb + so));
    st16(a.v_out + d, ld16(vb + so));
  }
}

}  // namespace

hipError_t launch_tokens(const TokenArgs &a, hipStream_t s) {
  const bool bf16 = a.elt == 2;
  if (a.n_dyn > 0) {
    if (bf16)
      hipLaunchKernelGGL(qsum_kernel<__bf16>, dim3(a.n_dyn), dim3(kSelThreads), 0, s, a);
    else
      hipLaunchKernelGGL(qsum_kernel<float>, dim3(a.n_dyn), dim3(kSelThreads), 0, s, a);
    if (a.n_cand > 0) {
      dim3 g((a.n_cand + 255) / 256, a.n_dyn);
      if (bf16)
        hipLaunchKernelGGL(phi_kernel<__bf16>, g, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL(phi_kernel<float>, g, dim3(256), 0, s, a);
    }
  }
  hipLaunchKernelGGL(token_select_kernel, dim3(a.H), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(gather_kernel, dim3((a.max_rows + 63) / 64, a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fkv
