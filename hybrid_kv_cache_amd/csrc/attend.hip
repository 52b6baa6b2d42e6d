// Attention of the current chunk's query block over a per-head KV range:
// the compressed, ragged cache (fkv_attend) or the whole uncompressed window
// (fkv_attend_dense).  Forcing-KV summary page (ai-feeds.com, arXiv
// 2605.09681), 方法 › 输出与工程收益: the compressed K/V replace the original
// cache in the layer's attention.  Non-causal: every query of the chunk sees
// every row of its head's range.
//
// bf16 kernel (D = 128): one workgroup = 4 waves x 32 queries of one head.
// K and V tiles of 64 keys are copied row-major from global memory straight
// into LDS (buffer loads with the LDS destination, double buffered, one
// barrier per tile, the next tiles' copies in flight during the current
// tile's math).  Scores S^T = K Q^T and the output O^T = V^T P^T run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the V^T operand comes
// straight from the row-major tile through transposing LDS reads.  Softmax
// in base 2 with the logit scale folded into one FMA per score.  The
// reference subtracted before exponentiation is the first tile's maximum and
// is raised (with a rescale of the accumulators) only when a tile's weight
// sum would pass 2^64: any reference gives the same normalised result, so
// the per-tile maximum and rescale are gone from the common path.
// Workgroups are spread so that each XCD (blockIdx % 8) runs a contiguous
// range of (head, query tile) pairs and shares that head's K/V in its L2.
#include "fkv_device.h"
#include "fkv_launch.h"

#include <type_traits>

namespace fkv {
namespace {

constexpr int kD = 128;
constexpr int kKT = 64;      // keys per tile
constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;
constexpr int kTileBytes = KvTileLds<kKT>::kBytes;
constexpr float kLazyRescale = 8.0f;         // log2 of the allowed growth (other kernels)

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
  // LDS: two K tiles and two V tiles, each its own array.  Step t (parity
  // P = t & 1) reads K(t+1) from sk[1-P] and V(t) from sv[P] while K(t+2) is
  // copied into sk[P] and V(t+1) into sv[1-P]; with the parity known at
  // compile time the compiler can see that the copies in flight never alias
  // the tiles being read, and does not wait for them.
  __shared__ __attribute__((aligned(1024))) char sk0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sk1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sv0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sv1[kTileBytes];
  typedef KvTileLds<kKT> Lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  // XCD-aware tile order: workgroups are handed to the 8 XCDs round-robin,
  // so workgroup b runs on XCD b % 8.  Give each XCD a contiguous range of
  // (head, query tile) pairs so that the workgroups sharing an L2 stream the
  // same head's K/V at the same time.
  const int ntq = (a.n_q + kBM - 1) / kBM;
  int h, qt;
  {
    const int nb = gridDim.x, b = blockIdx.x;
    const int x = b & 7, slot = b >> 3;
    const int pair = x * (nb >> 3) + min(x, nb & 7) + slot;
    h = pair / ntq;
    qt = pair - h * ntq;
  }
  const int qi = qt * kBM + wave * 32 + col;
  const KvView kv = kv_view(a, h);
  const int64_t rs_bytes = kv.rs * 2;

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
  const float c = a.c;

  // Staging: wave w fills tile rows 16 w .. 16 w + 15, four rows per
  // instruction; lane i lands at row 16 w + 4 j + i/16, chunk position i%16,
  // so it fetches global chunk (i%16) ^ swz(row) of that row.  Copies go
  // through buffer resources that end at the head's last row: rows past the
  // end of the range read as zeros (finite V where P is 0).  The tile offset
  // is a scalar, the lane offsets fixed.
  const int lrow = lane >> 4, lpos = lane & 15;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t range_bytes = (uint32_t)((int64_t)(kv.len - 1) * rs_bytes + kD * 2);
  const buf_rsrc krsrc = make_rsrc(kv.k, range_bytes);
  const buf_rsrc vrsrc = make_rsrc(kv.v, range_bytes);
  uint32_t goff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * wave + 4 * j + lrow;
    goff[j] = (uint32_t)row * (uint32_t)rs_bytes + ((lpos ^ Lds::swz(row)) << 4);
  }
  auto issue = [&](const buf_rsrc &rsrc, int it, char *dst) {
    const uint32_t soff = (uint32_t)((int64_t)it * kKT * rs_bytes);
    char *dw = dst + wave_s * (16 * 256);
#pragma unroll
    for (int j = 0; j < 4; ++j) buffer_load_lds16(rsrc, goff[j], soff, dw + j * 1024);
  };

  // V^T fragment addresses for the transposing reads (tile-relative): lane
  // group G = lane/16 reads rows 16 ks + 8 half + 4 g + j, columns
  // 32 db + 16 (G & 1) + 4 (lane & 3) .. +3.  The row part 16 ks + 8 half only
  // adds a constant, so one base per (db, half) serves every ks.
  const int tj = (lane & 15) >> 2, tc = lane & 3, tG = lane >> 4;
  uint32_t vbase[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 8 * half + 4 * g + tj;
      const int colv = 32 * db + 16 * (tG & 1) + 4 * tc;
      vbase[db][half] = Lds::offset(row, colv >> 3) + ((colv & 7) << 1);
    }
  // K fragment addresses: row kb*32 + col, chunk 2 st + g.
  uint32_t kbase[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) kbase[st] = Lds::offset(col, 2 * st + g);

  // S^T = K Q^T for one 64-key tile: 16 fragment reads feed 16 MFMAs on two
  // independent accumulators.
  auto qk = [&](const char *kl, f32x16 *sacc) {
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
    u32x4 kf[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) kf[i] = lds_read_b128(kl, kbase[i >> 1] + (i & 1) * 32 * 256);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      sacc[i & 1] = mfma32x32x16(__builtin_bit_cast(bf16x8, kf[i]), qf[i >> 1], sacc[i & 1]);
  };

  const int ntiles = (kv.len + kKT - 1) / kKT;
  // One tile step: softmax of this tile's scores `sc` (computed one step
  // earlier), next tile's scores into `sn`, then O += P V for this tile.
  // `par` is the step's parity as a compile-time constant.
  auto step = [&](auto par, int it, f32x16 *sc, f32x16 *sn) {
    constexpr int P = decltype(par)::value;
    char *const k_read = P ? sk0 : sk1;     // K(it+1)
    char *const k_fill = P ? sk1 : sk0;     // K(it+2)
    char *const v_read = P ? sv1 : sv0;     // V(it)
    char *const v_fill = P ? sv0 : sv1;     // V(it+1)
    wait_vmcnt0();   // K(it+1) and V(it), issued one step ago
    lds_barrier();
    if (it + 2 < ntiles) issue(krsrc, it + 2, k_fill);
    if (it + 1 < ntiles) issue(vrsrc, it + 1, v_fill);
    const int valid = kv.len - it * kKT;
    if (valid < kKT) {  // ragged last tile: keys past the end get no weight
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= valid) sc[kb][r] = -INFINITY;
        }
    }
    // Exact maximum of this tile's scaled scores (lane pair combined).
    auto tile_max = [&]() {
      float mx0 = sc[0][0], mx1 = sc[1][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        mx0 = fmaxf(mx0, sc[0][r]);
        mx1 = fmaxf(mx1, sc[1][r]);
      }
      return pair_max(fmaxf(mx0, mx1)) * c;
    };
    // Weights p = 2^(c s - m) of this tile as bf16 P^T fragments (k-step ks
    // covers keys 16 ks .. 16 ks + 15), and their sum as the PV product
    // sees them.
    bf16x8 pf[4];
    float lt = 0.f;
    auto weights = [&]() {
      const float nm = -m;
      lt = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kb = ks >> 1, base = (ks & 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 p2 = pack_bf16(fast_exp2(fmaf(sc[kb][base + e], c, nm)),
                                      fast_exp2(fmaf(sc[kb][base + e + 1], c, nm)));
          lt = __builtin_amdgcn_fdot2_f32_bf16(p2, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, lt, false);
          pf[ks][e] = p2[0];
          pf[ks][e + 1] = p2[1];
        }
      }
    };
    // The reference m is the first tile's maximum and is raised only when a
    // tile's weights sum past 2^64 (or overflow).  Any common reference gives
    // the same O / l, so skipping the per-tile maximum changes nothing
    // exactly, and weights up to 2^64 are far from fp32 / bf16 overflow.
    if (it == 0) m = tile_max();

    // Next tile's scores (independent of this tile's softmax).  On the last
    // step this reads a stale buffer and the result is never used; it stays
    // unconditional so that the MFMAs can interleave with the softmax.
    qk(k_read, sn);
    weights();
    // K-fragment reads run four ahead of the 16 score MFMAs of the next
    // tile, each followed by a slice of this tile's softmax.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
    if (__any(!(lt <= 0x1p64f))) {
      const float mnew = fmaxf(m, tile_max());
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      weights();
    }
    l += lt;

    // O^T += V^T P^T; lane (d = 32 db + col, g) receives keys 16 ks + 4 g + 0..3
    // and 16 ks + 8 + 4 g + 0..3, the key order of pf.
    const char *vl = v_read;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x2 lo = lds_read_tr16(vl, vbase[db][0] + 16 * 256 * ks);
        const u32x2 hi = lds_read_tr16(vl, vbase[db][1] + 16 * 256 * ks);
        const u32x4 raw = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, raw), pf[ks], o[db]);
      }
    }
    // PV: transposing reads two fragments ahead of the 16 MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 14; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  issue(krsrc, 0, sk0);
  issue(vrsrc, 0, sv0);
  if (ntiles > 1) issue(krsrc, 1, sk1);
  wait_vmcnt0();
  lds_barrier();
  f32x16 sa[2], sb[2];
  qk(sk0, sa);
  // Two steps per trip: the parity is static and the two score buffers swap
  // roles without copies.
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it, sa, sb);
    step(std::integral_constant<int, 1>{}, it + 1, sb, sa);
  }
  if (it < ntiles) step(std::integral_constant<int, 0>{}, it, sa, sb);

  const float lt = pair_sum(l);
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
  dim3 grid(((a.n_q + kBM - 1) / kBM) * a.H);
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
