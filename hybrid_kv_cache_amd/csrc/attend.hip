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

#include <atomic>
#include <type_traits>

namespace fkv {
namespace {

constexpr int kD = 128;
constexpr int kKT = 64;      // keys per tile
constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;
constexpr int kTileBytes = KvTileLds<kKT>::kBytes;
constexpr int kPartFloats = kBM * kD + 2 * kBM;  // one partial-result slot

struct KvView {
  const __bf16 *k;
  const __bf16 *v;
  int64_t rs;   // row stride in elements
  int len;
};

__device__ __forceinline__ KvView kv_view(const AttendArgs &a, int h) {
  KvView r;
  if (a.n_sel > 0 || a.tok_off) {
    const int64_t lo = a.n_sel > 0 ? a.host_off[h] : a.tok_off[h];
    const int64_t hi = a.n_sel > 0 ? a.host_off[h + 1] : a.tok_off[h + 1];
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

__device__ __forceinline__ int head_tiles(const AttendArgs &a, int h) {
  const int64_t len = a.n_sel > 0 ? a.host_off[h + 1] - a.host_off[h]
                      : a.tok_off ? a.tok_off[h + 1] - a.tok_off[h]
                                  : (int64_t)a.dense_len;
  return (int)((len + kKT - 1) / kKT);
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
  const float c = a.c;
  const int ntq = (a.n_q + kBM - 1) / kBM;
  const int pairs = ntq * (a.n_sel > 0 ? a.n_sel : a.H);
  // Work: (head, 128-query tile) pairs, p = h * ntq + qt (h the position in
  // sel for a head subset), pair p holding the
  // tiles(h) key tiles of its head.  Workgroups are handed to the 8 XCDs
  // round-robin (workgroup b runs on XCD b % 8); each XCD takes a contiguous
  // run of pairs, so the workgroups sharing an L2 stream the same head's K/V
  // at the same time.
  //  - Without a partial-result buffer: one whole pair per workgroup.
  //  - With one (fewer pairs than workgroups, all resident): the split
  //    schedule of xcd_split; a pair cut into a main part and a tail leaves
  //    two partial results for the combine kernel.
  //  - With one and more pairs than resident workgroups: the rounds
  //    schedule of xcd_rounds; its halved pairs leave two partial results
  //    in slots 2 (x cut_max + c) and 2 (x cut_max + c) + 1.
  const AttendWork wk = attend_work(pairs, a.part != nullptr, a.sched, a.slots_x, a.cut_max,
                                    gridDim.x, blockIdx.x);
  if (wk.n_items < 0) return;  // padding: XCDs with fewer pairs
  const int p0 = wk.p0, n_items = wk.n_items, k = wk.k, tail = wk.tail, slot0 = wk.slot0;
  const int64_t rs_bytes = (a.tok_off ? (int64_t)kD : a.kv_row_stride) * 2;

  // Staging: wave w fills tile rows 16 w .. 16 w + 15, four rows per
  // instruction; lane i lands at row 16 w + 4 j + i/16, chunk position i%16,
  // so it fetches global chunk (i%16) ^ swz(row) of that row.  Copies go
  // through buffer resources that end at the head's last row: rows past the
  // end of the range read as zeros (finite V where P is 0).  The tile offset
  // is a scalar, the lane offsets fixed.
  const int lrow = lane >> 4, lpos = lane & 15;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  // goff[j] carries -j KiB for the copy's immediate offset (row 16 w + 4 j
  // starts at least j KiB into the tile, so it stays non-negative).
  uint32_t goff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * wave + 4 * j + lrow;
    goff[j] = (uint32_t)row * (uint32_t)rs_bytes + ((lpos ^ Lds::swz(row)) << 4) - 1024u * j;
  }
  auto issue = [&](const buf_rsrc &rsrc, int it, char *dst) {
    const uint32_t soff = (uint32_t)((int64_t)it * kKT * rs_bytes);
    buffer_load_lds16x4(rsrc, goff, soff, dst + wave_s * (16 * 256));
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

  for (int item = 0; item < n_items; ++item) {
  const int p = p0 + item;
  const int hs = p / ntq, qt = p - hs * ntq;
  const int h = a.n_sel > 0 ? __builtin_amdgcn_readfirstlane(a.sel[hs]) : hs;
  const int nt = head_tiles(a, h);
  const int ts = k < 0 ? nt / 2 : split_tile(nt, k);
  const int t0 = tail ? ts : 0, t1 = tail ? nt : ts;
  if (t0 >= t1) continue;
  const int qi = qt * kBM + wave * 32 + col;
  const KvView kv = kv_view(a, h);
  const uint32_t range_bytes = (uint32_t)((int64_t)(kv.len - 1) * rs_bytes + kD * 2);
  const buf_rsrc krsrc = make_rsrc(kv.k, range_bytes);
  const buf_rsrc vrsrc = make_rsrc(kv.v, range_bytes);

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
    if (it + 2 < t1) issue(krsrc, it + 2, k_fill);
    if (it + 1 < t1) issue(vrsrc, it + 1, v_fill);
    const int valid = kv.len - it * kKT;
    if (valid < kKT) {  // ragged last tile: keys past the end get no weight
      // key = kb * 32 + 8 (r >> 2) + (r & 3) + 4 g: the lane's part moves to
      // the bound, so each test compares a constant with one register.
      const int bound = valid - 4 * g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) >= bound) sc[kb][r] = -INFINITY;
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
    if (it == t0) m = tile_max();

    // Next tile's scores (independent of this tile's softmax).  On the last
    // step this reads a stale buffer and the result is never used; it stays
    // unconditional so that the MFMAs can interleave with the softmax.
    // Issue priority 1 while this wave feeds the score MFMAs and the softmax,
    // back to 0 for the value product: the two waves sharing a SIMD take
    // turns instead of the older one running ahead.
    __builtin_amdgcn_s_setprio(1);
    qk(k_read, sn);
    weights();
    // K-fragment reads run four ahead of the 16 score MFMAs of the next
    // tile, each followed by a slice of up to eight of this tile's softmax
    // instructions (the softmax is spent by the last few MFMAs).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
    __builtin_amdgcn_s_setprio(0);
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

  issue(krsrc, t0, sk0);
  issue(vrsrc, t0, sv0);
  if (t0 + 1 < t1) issue(krsrc, t0 + 1, sk1);
  wait_vmcnt0();
  lds_barrier();
  f32x16 sa[2], sb[2];
  qk(sk0, sa);
  // Two steps per trip: the parity (counted from t0) is static and the two
  // score buffers swap roles without copies.
  int it = t0;
  for (; it + 1 < t1; it += 2) {
    step(std::integral_constant<int, 0>{}, it, sa, sb);
    step(std::integral_constant<int, 1>{}, it + 1, sb, sa);
  }
  if (it < t1) step(std::integral_constant<int, 0>{}, it, sa, sb);

  if (t0 == 0 && t1 == nt) {
    // Whole pair: normalise and store.
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
          bf16x2 hi2 = pack_bf16(o[db][4 * rr + 2] * inv, o[db][4 * rr + 3] * inv);
          u32x2 w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi2)};
          *reinterpret_cast<u32x2 *>(op + d0) = w;
        }
      }
    }
  } else {
    // Part of a pair: partial results into slot 2 p (main part) or
    // 2 p + 1 (tail); for a halved pair of the rounds schedule, slot0 or
    // slot0 + 1.
    float *slot = a.part + (int64_t)((slot0 >= 0 ? slot0 : 2 * p) + tail) * kPartFloats;
    const int ql = wave * 32 + col;
    const float lt = pair_sum(l);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = db * 32 + 8 * rr + 4 * g;
        f32x4 w = {o[db][4 * rr], o[db][4 * rr + 1], o[db][4 * rr + 2], o[db][4 * rr + 3]};
        *reinterpret_cast<f32x4 *>(slot + ql * kD + d0) = w;
      }
    if (g == 0) {
      slot[kBM * kD + ql] = m;
      slot[kBM * kD + kBM + ql] = lt;
    }
  }

  // The next item refills the LDS tiles: every wave must be done with
  // this one's.
  lds_barrier();
  }
}

// Merge of the two halves of every cut pair (block p: pair p):
// O = sum_s O_s 2^(m_s - M), l = sum_s l_s 2^(m_s - M), M = max_s m_s,
// out = O / l.  Thread t: query t / 2 of the tile, dims 64 (t & 1) .. +63.
// Split schedule: block p merges pair p.  Rounds schedule: block b merges
// the halved pair c = b / 8 of XCD x = b % 8 (if there is one).
__global__ __launch_bounds__(256) void attend_combine_kernel(AttendArgs a) {
  const int ntq = (a.n_q + kBM - 1) / kBM;
  const int pairs = ntq * a.H;
  int p, nt, ts, slot;
  if (a.sched == 2) {
    const int x = blockIdx.x & 7, c = blockIdx.x >> 3;
    const XcdRounds xr = xcd_rounds(pairs, a.slots_x, x);
    if (c >= xr.s) return;
    p = xr.p_lo + xr.w + c;
    nt = head_tiles(a, p / ntq);
    ts = nt / 2;
    slot = 2 * (x * a.cut_max + c);
  } else {
    p = blockIdx.x;
    int x = 0;
    while (x < 7 && p >= pairs * (x + 1) / 8) ++x;
    const XcdSplit sp = xcd_split(pairs, a.n_wg, x);
    nt = head_tiles(a, p / ntq);
    ts = split_tile(nt, sp.k);
    slot = 2 * p;
  }
  const int h = p / ntq, qt = p - h * ntq;
  if (ts == 0 || ts == nt) return;  // written whole by one workgroup

  const int t = threadIdx.x, ql = t >> 1, d0 = (t & 1) * 64;
  const float *s0 = a.part + (int64_t)slot * kPartFloats;
  const float *s1 = s0 + kPartFloats;
  const float m0 = s0[kBM * kD + ql], m1 = s1[kBM * kD + ql];
  const float M = fmaxf(m0, m1);
  const float f0 = fast_exp2(m0 - M), f1 = fast_exp2(m1 - M);
  const float L = s0[kBM * kD + kBM + ql] * f0 + s1[kBM * kD + kBM + ql] * f1;
  const f32x4 *x0 = reinterpret_cast<const f32x4 *>(s0 + ql * kD + d0);
  const f32x4 *x1 = reinterpret_cast<const f32x4 *>(s1 + ql * kD + d0);
  float acc[64];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const f32x4 u = x0[jj], v = x1[jj];
    acc[4 * jj] = u[0] * f0 + v[0] * f1;
    acc[4 * jj + 1] = u[1] * f0 + v[1] * f1;
    acc[4 * jj + 2] = u[2] * f0 + v[2] * f1;
    acc[4 * jj + 3] = u[3] * f0 + v[3] * f1;
  }
  const int qi = qt * kBM + ql;
  if (qi >= a.n_q) return;
  const float inv = 1.f / L;
  __bf16 *op = reinterpret_cast<__bf16 *>(a.out) + ((int64_t)qi * a.H + h) * kD + d0;
#pragma unroll
  for (int j = 0; j < 64; j += 4) {
    bf16x2 lo = pack_bf16(acc[j] * inv, acc[j + 1] * inv);
    bf16x2 hi2 = pack_bf16(acc[j + 2] * inv, acc[j + 3] * inv);
    u32x2 w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi2)};
    *reinterpret_cast<u32x2 *>(op + j) = w;
  }
}

// fp32 path (small shapes): a workgroup of 4 waves takes 64 queries of one
// head, one query per lane; wave w walks the keys w, w + 4, w + 8, ... of
// each 32-key tile staged in LDS (exact online softmax per key), and the four
// partial states (m, l, o) are merged in wave order at the end.
template <int D>
__global__ __launch_bounds__(256) void attend_f32_kernel(AttendArgs a) {
  constexpr int KT = 32, W = 4;
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  __shared__ float part_o[W - 1][64][D + 1];
  __shared__ float part_ml[W - 1][64][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y;
  const int qi = blockIdx.x * 64 + lane;
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
    for (int idx = tid; idx < KT * D; idx += 256) {
      const int j = idx / D, d = idx % D;
      ks[j][d] = j < n ? kb[(t0 + j) * rs + d] : 0.f;
      vs[j][d] = j < n ? vb[(t0 + j) * rs + d] : 0.f;
    }
    __syncthreads();
    for (int j = wave; j < n; j += W) {
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
  if (wave > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) part_o[wave - 1][lane][d] = o[d];
    part_ml[wave - 1][lane][0] = m;
    part_ml[wave - 1][lane][1] = l;
  }
  __syncthreads();
  if (wave == 0 && qi < a.n_q) {
    for (int w = 0; w < W - 1; ++w) {
      const float m2 = part_ml[w][lane][0], l2 = part_ml[w][lane][1];
      const float mn = fmaxf(m, m2);
      const float f1 = fast_exp2(m - mn), f2 = fast_exp2(m2 - mn);
      l = l * f1 + l2 * f2;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = o[d] * f1 + part_o[w][lane][d] * f2;
      m = mn;
    }
    float *op = reinterpret_cast<float *>(a.out) + ((int64_t)qi * a.H + h) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  }
}

}  // namespace

namespace {
// Compute units of the current device, looked up once per device: the
// attention calls ask for it on every launch.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 0;
  if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}
}  // namespace

size_t attend_part_bytes() {
  return (size_t)2 * 2 * device_cus() * kPartFloats * sizeof(float);
}

// Schedule of an attention launch over all heads (the sched field; the bf16
// and the fp8 kernel both run two workgroups per CU): 1 (split) with a
// partial-result buffer and at most one pair per CU; 2 (rounds) with one and
// more pairs than resident workgroups when some pairs are left for a last
// round; else 0, one workgroup per pair.  Fills the schedule fields of a and
// returns the combine kernel's workgroups (0: none).
int plan_attend(AttendArgs &a, void *part, size_t part_bytes) {
  const int pairs = ((a.n_q + kBM - 1) / kBM) * a.H;
  // Two workgroups fit on a CU (64 KiB of LDS each).  The split schedule
  // runs exactly that many, all resident at once, when there is at most one
  // pair per CU.  With more pairs than resident workgroups, whole pairs are
  // dealt out in rounds and the remainder halved so that the last round is
  // full too (xcd_rounds); the halves need 2 slots each, at most nb / 2 of
  // them.
  const int nb = 2 * device_cus();
  a.part = nullptr;
  a.n_wg = pairs;
  a.sched = 0;
  a.slots_x = 0;
  a.cut_max = 0;
  const bool have_part = part && nb > 0 && nb % 8 == 0 &&
                         part_bytes >= (size_t)2 * nb * kPartFloats * sizeof(float);
  if (have_part && 2 * pairs <= nb) {
    a.part = static_cast<float *>(part);
    a.n_wg = nb;
    a.sched = 1;
    return pairs;
  }
  if (have_part && pairs > nb) {
    int cut_max = 0, per_x = 0;
    for (int x = 0; x < 8; ++x) {
      const XcdRounds xr = xcd_rounds(pairs, nb / 8, x);
      cut_max = xr.s > cut_max ? xr.s : cut_max;
      per_x = xr.w + 2 * xr.s > per_x ? xr.w + 2 * xr.s : per_x;
    }
    if (cut_max > 0) {
      a.part = static_cast<float *>(part);
      a.n_wg = 8 * per_x;
      a.sched = 2;
      a.slots_x = nb / 8;
      a.cut_max = cut_max;
      return 8 * cut_max;
    }
  }
  return 0;
}

hipError_t launch_attend_combine(const AttendArgs &a, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(attend_combine_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

int attend_bf16_schedule(const AttendArgs &a0, void *part, size_t part_bytes) {
  AttendArgs a = a0;
  plan_attend(a, part, part_bytes);
  return a.sched;
}

hipError_t launch_attend_bf16(const AttendArgs &a0, void *part, size_t part_bytes,
                              hipStream_t s) {
  if (a0.D != kD) return hipErrorInvalidValue;
  AttendArgs a = a0;
  const int combine_blocks = plan_attend(a, part, part_bytes);
  hipLaunchKernelGGL(attend_bf16_kernel, dim3(a.n_wg), dim3(256), 0, s, a);
  if (combine_blocks > 0)
    hipLaunchKernelGGL(attend_combine_kernel, dim3(combine_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attend_bf16_heads(const AttendArgs &a0, hipStream_t s) {
  if (a0.D != kD || a0.n_sel <= 0 || a0.n_sel > kMaxHeads) return hipErrorInvalidValue;
  AttendArgs a = a0;
  a.part = nullptr;
  a.sched = 0;
  a.n_wg = ((a.n_q + kBM - 1) / kBM) * a.n_sel;
  hipLaunchKernelGGL(attend_bf16_kernel, dim3(a.n_wg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attend_f32(const AttendArgs &a, hipStream_t s) {
  dim3 grid((a.n_q + 63) / 64, a.H);
  if (a.D == 64)
    hipLaunchKernelGGL(attend_f32_kernel<64>, grid, dim3(256), 0, s, a);
  else if (a.D == 128)
    hipLaunchKernelGGL(attend_f32_kernel<128>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fkv
