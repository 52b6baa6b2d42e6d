// Dynamic-head segment scoring, first stage: per (sampled query, window
// frame) log-sum-exp of the scaled logits.  Forcing-KV summary page
// (ai-feeds.com, arXiv 2605.09681), 方法 › 关键模块 › 3 (dynamic similarity
// pruning): the history cache is grouped by frame and each group is scored
// by its attention with the current chunk's queries.  The score of a frame
// is the softmax mass it receives, so this stage reduces each frame's T
// logits to one log-sum-exp; the selection kernel then turns the per-frame
// values of one query into masses (a softmax over frames) and averages them.
//
// Splitting per frame keeps every frame's sum in a fixed order inside one
// workgroup, and makes equal logits give bit-identical per-frame values
// (with all logits 0, every frame's value is exactly log2(T)).
//
// bf16 kernel: workgroup = 4 waves x 32 sampled queries, one frame of one
// dynamic head; K rows of the frame stream through LDS in tiles of 64;
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16.
#include "fkv_device.h"
#include "fkv_launch.h"

namespace fkv {
namespace {

constexpr int kD = 128;
constexpr int kKT = 64;
constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;
constexpr int kKBytes = KvTileLds<kKT>::kBytes;

__global__ __launch_bounds__(256, 2) void score_bf16_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kKBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int di = blockIdx.z;
  const int h = a.dyn_heads[di];
  const int f = blockIdx.y;
  const int r = blockIdx.x * kBM + wave * 32 + col;   // sampled row
  const int64_t hd = (int64_t)a.H * kD;

  bf16x8 qf[8];
  if (r < a.n_s) {
    const int64_t qi = (int64_t)r * a.stride;
    const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) + qi * hd + (int64_t)h * kD + 8 * g;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8 *>(qp + 16 * st);
  } else {
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = bf16x8{};
  }

  const __bf16 *kb = reinterpret_cast<const __bf16 *>(a.k) + (int64_t)f * a.T * hd + (int64_t)h * kD;
  const int len = a.T;
  const int sc = tid & 15, sr = tid >> 4;
  u32x4 kr[4];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = t0 + sr + 16 * i;
      kr[i] = key < len ? ld16(kb + key * hd + sc * 8) : u32x4{0, 0, 0, 0};
    }
  };

  float m = kNegBig, l = 0.f;
  const int ntiles = (len + kKT - 1) / kKT;
  load_tile(0);
  for (int it = 0; it < ntiles; ++it) {
    char *kl = smem + (it & 1) * kKBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4 *>(kl + KvTileLds<kKT>::offset(sr + 16 * i, sc)) = kr[i];
    __syncthreads();
    if (it + 1 < ntiles) load_tile((it + 1) * kKT);
    const int valid = len - it * kKT;

    f32x16 s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      s[kb2] = f32x16{};
      const int row = kb2 * 32 + col;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        u32x4 raw = lds_read_b128(kl, KvTileLds<kKT>::offset(row, 2 * st + g));
        s[kb2] = mfma32x32x16(__builtin_bit_cast(bf16x8, raw), qf[st], s[kb2]);
      }
    }
    float mx = kNegBig;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int key = kb2 * 32 + 8 * (q >> 2) + 4 * g + (q & 3);
        float x = s[kb2][q] * a.c;
        x = key < valid ? x : -INFINITY;
        s[kb2][q] = x;
        mx = fmaxf(mx, x);
      }
    }
    const float mnew = fmaxf(m, mx);
    float ls = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int q = 0; q < 16; ++q) ls += fast_exp2(s[kb2][q] - mnew);
    }
    l = l * fast_exp2(m - mnew) + ls;
    m = mnew;
  }
  // Combine the two lanes that share a query column.
  const float m2 = swap_halves(m), l2 = swap_halves(l);
  const float M = fmaxf(m, m2);
  const float L = l * fast_exp2(m - M) + l2 * fast_exp2(m2 - M);
  if (g == 0 && r < a.n_s) a.lse[((int64_t)di * a.n_s + r) * a.F_tot + f] = M + fast_log2(L);
}

// fp32 path (small shapes): one workgroup per (sampled query, dynamic head);
// threads stride over each frame's keys, then a block reduction per frame.
template <int D>
__global__ __launch_bounds__(256) void score_f32_kernel(ScoreArgs a) {
  __shared__ float qs[D];
  __shared__ float red_m[4], red_l[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x, di = blockIdx.y;
  const int h = a.dyn_heads[di];
  const int64_t hd = (int64_t)a.H * D;
  const float *qp = reinterpret_cast<const float *>(a.q) + (int64_t)r * a.stride * hd + (int64_t)h * D;
  for (int d = tid; d < D; d += 256) qs[d] = qp[d];
  __syncthreads();
  const float *kbase = reinterpret_cast<const float *>(a.k) + (int64_t)h * D;
  for (int f = 0; f < a.F_tot; ++f) {
    float m = kNegBig, l = 0.f;
    for (int j = tid; j < a.T; j += 256) {
      const float *kp = kbase + ((int64_t)f * a.T + j) * hd;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qs[d], kp[d], s);
      const float x = s * a.c;
      const float mnew = fmaxf(m, x);
      l = l * fast_exp2(m - mnew) + fast_exp2(x - mnew);
      m = mnew;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float m2 = __shfl_xor(m, off, 64), l2 = __shfl_xor(l, off, 64);
      const float M = fmaxf(m, m2);
      l = l * fast_exp2(m - M) + l2 * fast_exp2(m2 - M);
      m = M;
    }
    if (lane == 0) {
      red_m[wave] = m;
      red_l[wave] = l;
    }
    __syncthreads();
    if (tid == 0) {
      float M = red_m[0], L = red_l[0];
      for (int w = 1; w < 4; ++w) {
        const float Mn = fmaxf(M, red_m[w]);
        L = L * fast_exp2(M - Mn) + red_l[w] * fast_exp2(red_m[w] - Mn);
        M = Mn;
      }
      a.lse[((int64_t)di * a.n_s + r) * a.F_tot + f] = M + fast_log2(L);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_score_bf16(const ScoreArgs &a, hipStream_t s) {
  if (a.D != kD) return hipErrorInvalidValue;
  dim3 grid((a.n_s + kBM - 1) / kBM, a.F_tot, a.n_dyn);
  hipLaunchKernelGGL(score_bf16_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_score_f32(const ScoreArgs &a, hipStream_t s) {
  dim3 grid(a.n_s, a.n_dyn);
  if (a.D == 64)
    hipLaunchKernelGGL(score_f32_kernel<64>, grid, dim3(256), 0, s, a);
  else if (a.D == 128)
    hipLaunchKernelGGL(score_f32_kernel<128>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fkv
