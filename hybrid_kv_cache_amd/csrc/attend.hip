// Attention of the current chunk's query block over a per-head KV range:
// the compressed, ragged cache (fkv_attend) or the whole uncompressed window
// (fkv_attend_dense).  Forcing-KV summary page (ai-feeds.com, arXiv
// 2605.09681), 方法 › 输出与工程收益: the compressed K/V replace the original
// cache in the layer's attention.  Non-causal: every query of the chunk sees
// every row of its head's range.
//
// bf16 kernel (D = 128): one workgroup = 4 waves x 32 queries of one head.
// K/V tiles of 64 keys are staged through LDS (double buffered, one barrier
// per tile, the next tile's global loads in flight during the current
// tile's math).  Scores S^T = K Q^T and the output O^T = V^T P^T run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the softmax is the online
// (running max / running sum) form in base 2 with the logit scale folded
// into the exponent.
#include "fkv_device.h"
#include "fkv_launch.h"

namespace fkv {
namespace {

constexpr int kD = 128;
constexpr int kKT = 64;      // keys per tile
constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;
constexpr int kKBytes = KTileLds<kKT>::kBytes;
constexpr int kVBytes = VtTileLds::kBytes;
constexpr int kStageBytes = kKBytes + kVBytes;

struct KvView {
  const __bf16 *k;
  const __bf16 *v;
  int64_t rs;   // row stride in elements
  int len;
};

__device__ __forceinline__ KvView kv_view(const AttendArgs &a, int h) {
  KvView r;
  if (a.tok_off) {
    const int64_t lo = a.tok_off[h], hi = a.tok_off[h + 1];
    r.k = reinterpret_cast<const __bf16 *>(a.k) + lo * kD;
    r.v = reinterpret_cast<const __bf16 *>(a.v) + lo * kD;
    r.rs = kD;
    r.len = (int)(hi - lo);
  } else {
    r.k = reinterpret_cast<const __bf16 *>(a.k) + (int64_t)h * kD;
    r.v = reinterpret_cast<const __bf16 *>(a.v) + (int64_t)h * kD;
    r.rs = a.kv_row_stride;
    r.len = a.dense_len;
  }
  return r;
}

__global__ __launch_bounds__(256, 2) void attend_bf16_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int h = blockIdx.y;
  const int qi = blockIdx.x * kBM + wave * 32 + col;
  const KvView kv = kv_view(a, h);

  // Q^T fragments (B operand of S^T = K Q^T): query qi, dims 16*st + 8*g ..
  bf16x8 qf[8];
  if (qi < a.n_q) {
    const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) + ((int64_t)qi * a.H + h) * kD + 8 * g;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8 *>(qp + 16 * st);
  } else {
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = bf16x8{};
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m = kNegBig, l = 0.f;

  // Staging: K rows (tid>>4) + 16 i, chunk tid&15; V rows 4*(tid>>4) + i,
  // chunk tid&15 (four consecutive keys per thread, transposed on the way
  // into LDS).
  const int sc = tid & 15, sr = tid >> 4;
  u32x4 kr[4], vr[4];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = t0 + sr + 16 * i;
      kr[i] = key < kv.len ? ld16(kv.k + key * kv.rs + sc * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = t0 + 4 * sr + i;
      vr[i] = key < kv.len ? ld16(kv.v + key * kv.rs + sc * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](char *kl, char *vl) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4 *>(kl + KTileLds<kKT>::offset(sr + 16 * i, sc)) = kr[i];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x2 lo = {pack_lo16(vr[0][w], vr[1][w]), pack_lo16(vr[2][w], vr[3][w])};
      u32x2 hi = {pack_hi16(vr[0][w], vr[1][w]), pack_hi16(vr[2][w], vr[3][w])};
      *reinterpret_cast<u32x2 *>(vl + VtTileLds::offset(8 * sc + 2 * w, sr)) = lo;
      *reinterpret_cast<u32x2 *>(vl + VtTileLds::offset(8 * sc + 2 * w + 1, sr)) = hi;
    }
  };

  const int ntiles = (kv.len + kKT - 1) / kKT;
  load_tile(0);
  for (int it = 0; it < ntiles; ++it) {
    char *kl = smem + (it & 1) * kStageBytes;
    char *vl = kl + kKBytes;
    store_tile(kl, vl);
    __syncthreads();
    if (it + 1 < ntiles) load_tile((it + 1) * kKT);
    const int valid = kv.len - it * kKT;

    // S^T for 64 keys x 32 queries: two 32x32 blocks.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int row = kb * 32 + col;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        u32x4 raw = lds_read_b128(kl, KTileLds<kKT>::offset(row, 2 * st + g));
        s[kb] = mfma32x32x16(__builtin_bit_cast(bf16x8, raw), qf[st], s[kb]);
      }
    }
    float mx = kNegBig;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        float x = s[kb][r] * a.c;
        x = key < valid ? x : -INFINITY;
        s[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, swap_halves(mx));
    const float mnew = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[kb][r] - m);
        ls += p;
        s[kb][r] = p;
      }
    }
    l += ls;

    // P^T fragments: k-step ks covers keys 16 ks .. 16 ks + 15 of the tile.
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1, base = (ks & 1) * 8;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        bf16x2 p2 = pack_bf16(s[kb][base + e], s[kb][base + e + 1]);
        pf[ks][e] = p2[0];
        pf[ks][e + 1] = p2[1];
      }
    }
    // O^T += V^T P^T; lane (d = 32 db + col, g) feeds keys 16 ks + 4 g + 0..3
    // and 16 ks + 8 + 4 g + 0..3, matching the key order of pf.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + col;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x2 lo = lds_read_b64(vl, VtTileLds::offset(d, 4 * ks + g));
        u32x2 hi = lds_read_b64(vl, VtTileLds::offset(d, 4 * ks + 2 + g));
        u32x4 raw = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, raw), pf[ks], o[db]);
      }
    }
  }

  const float lt = l + swap_halves(l);
  const float inv = 1.f / lt;
  if (qi < a.n_q) {
    __bf16 *op = reinterpret_cast<__bf16 *>(a.out) + ((int64_t)qi * a.H + h) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = db * 32 + 8 * rr + 4 * g;
        bf16x2 lo = pack_bf16(o[db][4 * rr] * inv, o[db][4 * rr + 1] * inv);
        bf16x2 hi = pack_bf16(o[db][4 * rr + 2] * inv, o[db][4 * rr + 3] * inv);
        u32x2 w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        *reinterpret_cast<u32x2 *>(op + d0) = w;
      }
    }
  }
}

// fp32 path (small shapes): one thread per query, keys staged 32 at a time in
// LDS and read by broadcast; exact online softmax per key.
template <int D>
__global__ __launch_bounds__(64) void attend_f32_kernel(AttendArgs a) {
  constexpr int KT = 32;
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int qi = blockIdx.x * 64 + tid;
  const float *kb, *vb;
  int64_t rs;
  int len;
  if (a.tok_off) {
    const int64_t lo = a.tok_off[h], hi = a.tok_off[h + 1];
    kb = reinterpret_cast<const float *>(a.k) + lo * D;
    vb = reinterpret_cast<const float *>(a.v) + lo * D;
    rs = D;
    len = (int)(hi - lo);
  } else {
    kb = reinterpret_cast<const float *>(a.k) + (int64_t)h * D;
    vb = reinterpret_cast<const float *>(a.v) + (int64_t)h * D;
    rs = a.kv_row_stride;
    len = a.dense_len;
  }
  float q[D], o[D];
  const float *qp = reinterpret_cast<const float *>(a.q) + ((int64_t)(qi < a.n_q ? qi : 0) * a.H + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qi < a.n_q ? qp[d] : 0.f;
    o[d] = 0.f;
  }
  float m = kNegBig, l = 0.f;
  for (int t0 = 0; t0 < len; t0 += KT) {
    const int n = min(KT, len - t0);
    for (int idx = tid; idx < KT * D; idx += 64) {
      const int j = idx / D, d = idx % D;
      ks[j][d] = j < n ? kb[(t0 + j) * rs + d] : 0.f;
      vs[j][d] = j < n ? vb[(t0 + j) * rs + d] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], ks[j][d], s);
      const float x = s * a.c;
      const float mnew = fmaxf(m, x);
      const float alpha = fast_exp2(m - mnew);
      const float p = fast_exp2(x - mnew);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, vs[j][d], o[d] * alpha);
      m = mnew;
    }
    __syncthreads();
  }
  if (qi < a.n_q) {
    float *op = reinterpret_cast<float *>(a.out) + ((int64_t)qi * a.H + h) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  }
}

}  // namespace

hipError_t launch_attend_bf16(const AttendArgs &a, hipStream_t s) {
  if (a.D != kD) return hipErrorInvalidValue;
  dim3 grid((a.n_q + kBM - 1) / kBM, a.H);
  hipLaunchKernelGGL(attend_bf16_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attend_f32(const AttendArgs &a, hipStream_t s) {
  dim3 grid((a.n_q + 63) / 64, a.H);
  if (a.D == 64)
    hipLaunchKernelGGL(attend_f32_kernel<64>, grid, dim3(64), 0, s, a);
  else if (a.D == 128)
    hipLaunchKernelGGL(attend_f32_kernel<128>, grid, dim3(64), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fkv
