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
//                  (fp32, rows in order);
//   phi_kernel     phi[j] = k_j . Qsum for every candidate token (one thread
//                  per token, fp32, dims in order) -- sum_r q_r . k_j regrouped;
//   token_select_kernel
//                  one workgroup per head: the kept history tokens in
//                  ascending order (static: pattern flags; dynamic: a 4-pass
//                  8-bit radix select finds the C-th largest phi, ties to the
//                  lower index), written as the window token index of every
//                  compacted row, plus the current chunk;
//   gather_kernel  copies the K and V rows those indices name.
#include "fkv_device.h"
#include "fkv_launch.h"

namespace fkv {
namespace {

constexpr int kSelThreads = 1024;

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }

template <typename T>
__global__ __launch_bounds__(128) void qsum_kernel(TokenArgs a) {
  const int di = blockIdx.x, h = a.dyn_heads[di];
  const int64_t hd = (int64_t)a.H * a.D;
  const T *q = reinterpret_cast<const T *>(a.q) + (int64_t)h * a.D;
  for (int d = threadIdx.x; d < a.D; d += blockDim.x) {
    float s = 0.f;
    for (int r = 0; r < a.n_q; r += a.stride) s += to_f32<T>(q[(int64_t)r * hd + d]);
    a.qsum[di * a.D + d] = s;
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

__device__ __forceinline__ bool static_keeps(const TokenArgs &a, int t) {
  if (t < a.sink_tok) return true;
  const int chunk = a.F_c * a.T;
  const int lo = (t / chunk) * chunk;
  const int hi = min(lo + chunk, a.n_hist);
  return t - lo < a.boundary || hi - t <= a.boundary;
}

__global__ __launch_bounds__(kSelThreads) void token_select_kernel(TokenArgs a) {
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
    // static pattern over the history, in token order
    for (int base = 0; base < a.n_hist; base += kSelThreads) {
      const int t = base + tid;
      const int keep = t < a.n_hist && static_keeps(a, t);
      int total;
      const int p = block_excl_scan(keep, wsum, &total);
      if (keep) out[pos + p] = t;
      pos += total;
    }
  } else {
    // sink zone
    for (int t = tid; t < a.sink_tok; t += kSelThreads) out[t] = t;
    pos = a.sink_tok;
    const float *phi = a.phi + (int64_t)di * a.n_cand;
    const int n = a.n_cand, c = min(a.budget, n);
    uint32_t thr = 0;
    int remaining = 0;  // keys equal to thr to take, lowest index first
    if (c > 0 && c < n) {
      // radix select of the c-th largest key, 8 bits per pass from the top
      uint32_t prefix = 0;
      int need = c;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (int j = tid; j < n; j += kSelThreads) {
          const uint32_t key = sort_key(phi[j]);
          const bool match = pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8));
          if (match) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        if (tid == 0) {
          int acc = 0, d = 255;
          for (; d > 0; --d) {
            if (acc + hist[d] >= need) break;
            acc += hist[d];
          }
          s_prefix = prefix | ((uint32_t)d << shift);
          s_remaining = need - acc;
        }
        __syncthreads();
        prefix = s_prefix;
        need = s_remaining;
        __syncthreads();
      }
      thr = prefix;
      remaining = need;
    }
    // kept candidates in index order: key > thr, or key == thr among the
    // first `remaining` such (all of them when c == n, none when c == 0)
    int eq_seen = 0;
    for (int base = 0; base < n; base += kSelThreads) {
      const int j = base + tid;
      bool gt = false, eq = false;
      if (j < n && c > 0) {
        if (c >= n) {
          gt = true;
        } else {
          const uint32_t key = sort_key(phi[j]);
          gt = key > thr;
          eq = key == thr;
        }
      }
      int eq_total;
      const int eq_rank = eq_seen + block_excl_scan(eq ? 1 : 0, wsum, &eq_total);
      eq_seen += eq_total;
      const int take = gt || (eq && eq_rank < remaining);
      int total;
      const int p = block_excl_scan(take, wsum, &total);
      if (take) out[pos + p] = a.cand_lo + j;
      pos += total;
    }
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
  const int v16 = row_bytes >> 4;
  const int64_t tm = (int64_t)a.H * row_bytes;
  const char *kb = reinterpret_cast<const char *>(a.k) + (int64_t)h * row_bytes;
  const char *vb = reinterpret_cast<const char *>(a.v) + (int64_t)h * row_bytes;
  for (int i = threadIdx.x; i < rows * v16; i += 256) {
    const int r = i / v16, p = i - r * v16;
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
      hipLaunchKernelGGL(qsum_kernel<__bf16>, dim3(a.n_dyn), dim3(128), 0, s, a);
    else
      hipLaunchKernelGGL(qsum_kernel<float>, dim3(a.n_dyn), dim3(128), 0, s, a);
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
