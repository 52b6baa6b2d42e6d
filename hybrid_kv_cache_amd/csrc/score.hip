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
// dynamic head; K rows of the frame are copied straight into a two-slot LDS
// ring in tiles of 64 (the next tile in flight while one is read; 32 KB of
// LDS, so four workgroups share a CU and hide the copies' latency -- deeper
// rings at two workgroups per CU measured 5-10% slower);
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16.  Frames are located through the
// window view: a plain token-major window, or a head's ragged history (a
// previous compressed cache) followed by the current chunk.  Head profiling
// runs the same kernel over every head with stride 1.
#include "fkv_device.h"
#include "fkv_launch.h"

namespace fkv {
namespace {

constexpr int kD = 128;
constexpr int kKT = 64;
constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;
constexpr int kTileBytes = KvTileLds<kKT>::kBytes;
constexpr int kAhead = 1;              // tiles in flight ahead of the one read (<= 3)
constexpr int kRing = kAhead + 1;

// Wait until at most `tiles` tile copies (4 loads each) of this wave remain
// in flight: s_waitcnt vmcnt(8 / 4 / 0), gfx9 encoding.
__device__ __forceinline__ void wait_tiles_in_flight(int tiles) {
  if (tiles >= 2)
    __builtin_amdgcn_s_waitcnt(0x0F78);
  else if (tiles == 1)
    __builtin_amdgcn_s_waitcnt(0x0F74);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

__global__ __launch_bounds__(256, 4) void score_bf16_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kRing * kTileBytes];
  typedef KvTileLds<kKT> Lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  // Work unit u = (dynamic head di, window frame f), u = di * F_tot + f,
  // split into n_qb blocks of 128 sampled queries that all read the frame's
  // K.  Workgroups go to the 8 XCDs round-robin (workgroup b runs on XCD
  // b % 8), so unit u is given to XCD u % 8 and its query blocks to
  // consecutive workgroups of that XCD: they run together and the frame's K
  // comes from HBM once, then from the XCD's L2.
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int lu = slot / a.n_qb, qb = slot - lu * a.n_qb;
  const int u = lu * 8 + xcd;
  if (u >= a.n_dyn * a.F_tot) return;  // padding of the last round of units
  const int di = u / a.F_tot;
  const int f = u - di * a.F_tot;
  // The head index is read from a kernel-argument array with a runtime
  // index; readfirstlane tells the compiler it is wave-uniform, so the K
  // buffer resource stays in scalar registers.
  const int h = __builtin_amdgcn_readfirstlane(a.dyn_heads[di]);
  const int fh_h = __builtin_amdgcn_readfirstlane(a.fh[h]);
  if (f >= fh_h + a.F_c) return;  // beyond this head's window
  const int r = qb * kBM + wave * 32 + col;   // sampled row
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

  // K rows of frame f of head h's window, rs_bytes apart.
  int64_t rs_bytes;
  const char *kframe = frame_rows(a.win, false, h, fh_h, f, a.T, &rs_bytes);
  const int len = a.T;
  const int ntiles = (len + kKT - 1) / kKT;
  const int lrow = lane >> 4, lpos = lane & 15;
  auto ring = [&](int t) { return smem + (t % kRing) * kTileBytes; };
  // Tile `it` -> LDS (4 direct copies per wave: rows 16 w + 4 j + lane/16).
  // Copies through a buffer resource ending at the frame's last row: rows
  // past the frame read as zeros (and are masked out of the sums).
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const buf_rsrc krsrc = make_rsrc(kframe, (uint32_t)((int64_t)(len - 1) * rs_bytes + kD * 2));
  // goff[j] carries -j KiB for the copy's immediate offset (row 16 w + 4 j
  // starts at least j KiB into the tile).
  uint32_t goff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * wave + 4 * j + lrow;
    goff[j] = (uint32_t)row * (uint32_t)rs_bytes + ((lpos ^ Lds::swz(row)) << 4) - 1024u * j;
  }
  auto issue = [&](int it) -> bool {
    if (it >= ntiles) return false;
    const uint32_t soff = (uint32_t)((int64_t)it * kKT * rs_bytes);
    buffer_load_lds16x4(krsrc, goff, soff, ring(it) + wave_s * (16 * 256));
    return true;
  };
  uint32_t kbase[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) kbase[st] = Lds::offset(col, 2 * st + g);

  for (int t = 0; t < kAhead; ++t) issue(t);
  float m = kNegBig, l = 0.f;
  // A wave whose 32 sampled rows all lie past the sample (the tail of the
  // last query block) keeps its share of the copies and barriers but skips
  // the arithmetic.
  const bool active = __builtin_amdgcn_readfirstlane(qb * kBM + wave * 32) < a.n_s;
  for (int it = 0; it < ntiles; ++it) {
    // Tile `it` must have landed; the (at most kAhead - 1) later ones may
    // stay in flight.
    wait_tiles_in_flight(min(kAhead - 1, ntiles - 1 - it));
    __syncthreads();
    issue(it + kAhead);
    if (!active) continue;
    const char *kl = ring(it);
    const int valid = len - it * kKT;

    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
    // Issue priority 1 while this wave reads its K fragments and feeds the
    // MFMAs, back to 0 for the softmax: the two waves sharing a SIMD take
    // turns, one's exponentials beside the other's MFMAs.
    __builtin_amdgcn_s_setprio(1);
    u32x4 kf[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) kf[i] = lds_read_b128(kl, kbase[i >> 1] + (i & 1) * 32 * 256);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      s[i & 1] = mfma32x32x16(__builtin_bit_cast(bf16x8, kf[i]), qf[i >> 1], s[i & 1]);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    __builtin_amdgcn_s_setprio(0);

    if (valid < kKT) {
      // key = kb * 32 + 8 (q >> 2) + (q & 3) + 4 g: the lane's part moves to
      // the bound, so each test compares a constant with one register.
      const int bound = valid - 4 * g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (kb * 32 + 8 * (q >> 2) + (q & 3) >= bound) s[kb][q] = -INFINITY;
    }
    // Per-lane running sum of 2^(c s - m).  The reference m is this lane's
    // first-tile maximum and is raised only when a tile's sum passes 2^64 (or
    // overflows): any reference gives the same log-sum-exp.
    auto lane_max = [&]() {
      float mx0 = s[0][0], mx1 = s[1][0];
#pragma unroll
      for (int q = 1; q < 16; ++q) {
        mx0 = fmaxf(mx0, s[0][q]);
        mx1 = fmaxf(mx1, s[1][q]);
      }
      return fmaxf(mx0, mx1) * a.c;
    };
    auto tile_sum = [&]() {
      const float nm = -m;
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        ls0 += fast_exp2(fmaf(s[0][q], a.c, nm));
        ls1 += fast_exp2(fmaf(s[1][q], a.c, nm));
      }
      return ls0 + ls1;
    };
    if (it == 0) m = fmaxf(lane_max(), kNegBig);
    float lt = tile_sum();
    if (__any(!(lt <= 0x1p64f))) {
      const float mnew = fmaxf(m, lane_max());
      l *= fast_exp2(m - mnew);
      m = mnew;
      lt = tile_sum();
    }
    l += lt;
  }
  // Combine the two lanes that share a query column.
  const float m2 = swap_halves(m), l2 = swap_halves(l);
  const float M = fmaxf(m, m2);
  const float L = l * fast_exp2(m - M) + l2 * fast_exp2(m2 - M);
  if (g == 0 && r < a.n_s) a.lse[((int64_t)di * a.F_tot + f) * a.n_s + r] = M + fast_log2(L);
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
  const int fh_h = a.fh[h];
  for (int f = 0; f < fh_h + a.F_c; ++f) {
    int64_t rs_bytes;
    const char *kframe = frame_rows(a.win, false, h, fh_h, f, a.T, &rs_bytes);
    float m = kNegBig, l = 0.f;
    for (int j = tid; j < a.T; j += 256) {
      const float *kp = reinterpret_cast<const float *>(kframe + j * rs_bytes);
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
      a.lse[((int64_t)di * a.F_tot + f) * a.n_s + r] = M + fast_log2(L);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_score_bf16(const ScoreArgs &a0, hipStream_t s) {
  if (a0.D != kD) return hipErrorInvalidValue;
  ScoreArgs a = a0;
  a.n_qb = (a.n_s + kBM - 1) / kBM;
  const int64_t units = (int64_t)a.n_dyn * a.F_tot;
  const int64_t blocks = (units + 7) / 8 * 8 * a.n_qb;
  if (units <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(score_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
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
