// FP8 (OCP e4m3) compressed cache: quantizing compaction and attention on
// v_mfma_f32_32x32x64_f8f6f4.  Forcing-KV summary page (ai-feeds.com, arXiv
// 2605.09681), 行业影响 › 与现有产品/工作流的接口: the method stacks with
// quantization to shrink the cache further.
//
// Quantization: code(x / scale[h]) -- an IEEE fp32 division, clamped to
// [-448, 448], then v_cvt_pk_fp8_f32 (round to nearest even).
//
// Attention workgroup: 4 waves x 32 queries of one head, 64-key tiles of
// 128-byte rows in LDS (K and V double-buffered, 8 KiB each).  The query
// fragment is quantized once per workgroup.  Scores S^T = K Q^T: per 64-key
// tile 2 key blocks x 2 dim steps of the 32x32x64 MFMA, whose A lane l holds
// row l % 32 and k-elements 32 (l / 32) .. +31 (bytes in order).  K rows are
// read in the permuted order sigma so that the accumulator of lane
// (query, g) ends up holding keys 32 g + 0 .. 31 in register order: the
// rounded weights then form the B operand of O^T += V^T P^T as they are,
// and V^T comes from the row-major tile through 8-bit transposing reads of
// 8 consecutive keys.  The row sums come from one more MFMA whose A holds
// ones in row 0, so they are the sums of exactly the fp8 weights the value
// product uses.  Softmax reference: the running maximum m is raised (and
// the accumulators rescaled) when a tile's maximum passes m + 8, so every
// weight 2^(s c - m) stays at most 2^8, inside e4m3's range.
#include "fkv_device.h"
#include "fkv_fp8.h"
#include "fkv_launch.h"

#include <type_traits>

namespace fkv {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kKT = 64;
constexpr int kBM = 128;
constexpr int kRow = 128;                 // bytes per fp8 row
constexpr int kTileBytes = kKT * kRow;    // 8 KiB
constexpr float kE4m3Max = 448.f;
constexpr int kPartFloats = kBM * kD + 2 * kBM;  // one partial-result slot (as bf16)

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Two fp32 -> two e4m3 bytes in the low (HI false) or high half of `old`.
template <bool HI>
__device__ __forceinline__ int cvt2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -kE4m3Max), kE4m3Max); }

// 16-byte chunk c of tile row r sits at chunk position c ^ swz8(r).  Keeps
// the K fragment reads (16 lanes: rows {r0..r0+7, r0+32..r0+39} in the
// permuted key order, one chunk) and the transposing V reads (32 lanes: 8
// aligned rows x 2 chunks) on distinct banks.
__device__ __forceinline__ uint32_t swz8(int r) {
  return (uint32_t)((((r >> 1) & 3) << 1) | (((r >> 3) ^ (r >> 5)) & 1));
}
__device__ __forceinline__ uint32_t tile_off(int r, int chunk) {
  return (uint32_t)(r * kRow) + (((uint32_t)chunk ^ swz8(r)) << 4);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const char *base, uint32_t off) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(base + off));
}

__global__ __launch_bounds__(256, 2) void attend_fp8_kernel(AttendFp8Args a) {
  __shared__ __attribute__((aligned(1024))) char sk0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sk1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sv0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sv1[kTileBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int ntq = (a.n_q + kBM - 1) / kBM;
  // Work: (head, 128-query tile) pairs p = h * ntq + qt, each XCD (workgroup
  // b runs on XCD b % 8) a contiguous run of them; with a partial-result
  // buffer the balanced schedules of the bf16 kernel (attend_work): pairs
  // cut into a main part and a tail, or the last round's pairs halved,
  // their partial results merged by the combine kernel.
  const AttendWork wk = attend_work(ntq * a.H, a.part != nullptr, a.sched, a.slots_x, a.cut_max,
                                    gridDim.x, blockIdx.x);
  if (wk.n_items < 0) return;  // padding: XCDs with fewer pairs
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);

  // Staging: wave w copies tile rows 16 w .. 16 w + 15, 8 rows per
  // instruction; lane i lands at row 16 w + 8 j + i / 8, chunk position i % 8,
  // fetching global chunk (i % 8) ^ swz8(row).  The buffer resource ends at
  // the head's last row (rows past it read as zeros).
  uint32_t goff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * wave + 8 * j + (lane >> 3);
    goff[j] = (uint32_t)row * kRow + (((lane & 7) ^ swz8(row)) << 4) - 1024u * j;
  }

  // K fragment addresses: A lane (row R = 32 kb + col, g) reads key
  // sigma(R) = 32 ((R >> 2) & 1) + 16 kb + 4 ((R >> 3) & 3) + (R & 3),
  // chunks 4 ds + 2 g and +1.
  uint32_t koff[2][2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int R = 32 * kb + col;
    const int key = 32 * ((R >> 2) & 1) + 16 * kb + 4 * ((R >> 3) & 3) + (R & 3);
#pragma unroll
    for (int ds = 0; ds < 2; ++ds)
#pragma unroll
      for (int e = 0; e < 2; ++e) koff[kb][ds][e] = tile_off(key, 4 * ds + 2 * g + e);
  }
  // V^T fragment addresses: lane group G = lane / 16, member s = lane % 16
  // supplies row 32 g + 8 t + s / 2 (t = 0 .. 3), byte column 32 db + 16 (G & 1)
  // + 8 (s % 2) .. +7; it receives column 32 db + col of rows 32 g + 8 t .. +7.
  const int G = lane >> 4, sm = lane & 15;
  uint32_t voff[4][4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = 32 * g + 8 * t + (sm >> 1);
      voff[db][t] = tile_off(row, 2 * db + (G & 1)) + 8 * (sm & 1);
    }
  // Row-sum operand: ones (0x38 = 1.0) in row 0 of A.
  i32x8 ones;
#pragma unroll
  for (int w = 0; w < 8; ++w) ones[w] = col == 0 ? 0x38383838 : 0;

  for (int item = 0; item < wk.n_items; ++item) {
  const int p = wk.p0 + item;
  const int h = p / ntq, qt = p - h * ntq;
  const int qi = qt * kBM + wave * 32 + col;
  const int64_t lo = a.tok_off[h], len64 = a.tok_off[h + 1] - lo;
  const int len = (int)len64;
  const int nt = (len + kKT - 1) / kKT;
  const int ts = wk.k < 0 ? nt / 2 : split_tile(nt, wk.k);
  const int t0 = wk.tail ? ts : 0, t1 = wk.tail ? nt : ts;
  if (t0 >= t1) continue;
  const float c = a.c * a.q_scale[h] * a.k_scale[h];

  // Query fragments: lane (query, g) holds dims 64 ds + 32 g + 0 .. 31 as
  // e4m3 codes of q / q_scale.
  i32x8 qf[2];
  {
    const float qs = a.q_scale[h];
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      qf[ds] = i32x8{};
      if (qi < a.n_q) {
        const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) +
                           ((int64_t)qi * a.H + h) * kD + 64 * ds + 32 * g;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          float f[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] = clamp448((float)qp[4 * w + e] / qs);
          int v = cvt2<false>(f[0], f[1], 0);
          v = cvt2<true>(f[2], f[3], v);
          qf[ds][w] = v;
        }
      }
    }
  }

  const char *kbase_g = reinterpret_cast<const char *>(a.k) + lo * kRow;
  const char *vbase_g = reinterpret_cast<const char *>(a.v) + lo * kRow;
  const uint32_t range_bytes = (uint32_t)(len64 * kRow);
  const buf_rsrc krsrc = make_rsrc(kbase_g, range_bytes);
  const buf_rsrc vrsrc = make_rsrc(vbase_g, range_bytes);
  auto issue = [&](const buf_rsrc &rsrc, int it, char *dst) {
    const uint32_t soff = (uint32_t)(it * kKT * kRow);
    char *dw = dst + wave_s * 2048;
    buffer_load_lds16<0>(rsrc, goff[0], soff, dw);
    buffer_load_lds16<1024>(rsrc, goff[1], soff, dw);
  };

  auto qk = [&](const char *kl, f32x16 *sacc) {
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) {
        const u32x4 x0 = lds_read_b128(kl, koff[kb][ds][0]);
        const u32x4 x1 = lds_read_b128(kl, koff[kb][ds][1]);
        const i32x8 af = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                          (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        sacc[kb] = mfma_fp8(af, qf[ds], sacc[kb]);
      }
  };

  f32x16 o[4], lsum;
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  lsum = f32x16{};
  float m = 0.f;

  auto step = [&](auto par, int it, f32x16 *sc, f32x16 *sn) {
    constexpr int P = decltype(par)::value;
    char *const k_read = P ? sk0 : sk1;     // K(it+1)
    char *const k_fill = P ? sk1 : sk0;     // K(it+2)
    char *const v_read = P ? sv1 : sv0;     // V(it)
    char *const v_fill = P ? sv0 : sv1;     // V(it+1)
    wait_vmcnt0();
    lds_barrier();
    if (it + 2 < t1) issue(krsrc, it + 2, k_fill);
    if (it + 1 < t1) issue(vrsrc, it + 1, v_fill);
    const int valid = len - it * kKT;
    if (valid < kKT) {
      // The lane's part of the key index (32 g) moves to the bound, so each
      // test compares a constant with one register.
      const int bound = valid - 32 * g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * kb + r >= bound) sc[kb][r] = -INFINITY;
    }
    // Reference: the first tile's maximum, raised whenever a tile's maximum
    // passes it by more than 8 (weights stay <= 2^8).
    float mx = sc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
    mx = pair_max(mx) * c;
    if (it == t0) {
      m = mx;
    } else if (__any(mx > m + 8.f)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      lsum *= alpha;
    }
    // Issue priority 1 for the score MFMAs and the softmax, 0 for the value
    // product (the waves sharing a SIMD take turns).
    __builtin_amdgcn_s_setprio(1);
    qk(k_read, sn);
    // Weights as e4m3 codes: byte i of the B operand = key 32 g + i.
    i32x8 pf;
    const float nm = -m;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float p0 = fast_exp2(fmaf(sc[kb][4 * t], c, nm));
        const float p1 = fast_exp2(fmaf(sc[kb][4 * t + 1], c, nm));
        const float p2 = fast_exp2(fmaf(sc[kb][4 * t + 2], c, nm));
        const float p3 = fast_exp2(fmaf(sc[kb][4 * t + 3], c, nm));
        int v = cvt2<false>(p0, p1, 0);
        pf[4 * kb + t] = cvt2<true>(p2, p3, v);
      }
    // Score MFMAs of the next tile interleaved with this tile's softmax:
    // K-fragment reads four ahead, then per MFMA one read and a slice of
    // the weights.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      i32x8 vf;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const i32x2 x = lds_read_tr8(v_read, voff[db][t]);
        vf[2 * t] = x[0];
        vf[2 * t + 1] = x[1];
      }
      o[db] = mfma_fp8(vf, pf, o[db]);
    }
    lsum = mfma_fp8(ones, pf, lsum);
    // Value product: transposing reads eight ahead, two per MFMA after that.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  };

  {
    issue(krsrc, t0, sk0);
    issue(vrsrc, t0, sv0);
    if (t0 + 1 < t1) issue(krsrc, t0 + 1, sk1);
    wait_vmcnt0();
    lds_barrier();
    f32x16 sa[2], sb[2];
    qk(sk0, sa);
    int it = t0;
    for (; it + 1 < t1; it += 2) {
      step(std::integral_constant<int, 0>{}, it, sa, sb);
      step(std::integral_constant<int, 1>{}, it + 1, sb, sa);
    }
    if (it < t1) step(std::integral_constant<int, 0>{}, it, sa, sb);
  }

  // Row sums sit in element 0 of the g = 0 lane of each query.
  const float l0 = lsum[0];
  const float l1 = swap_halves(l0);
  const float l = g == 0 ? l0 : l1;
  if (t0 == 0 && t1 == nt) {
    // Whole pair: normalise and store.
    const float f = a.v_scale[h] / l;
    if (qi < a.n_q) {
      __bf16 *op = reinterpret_cast<__bf16 *>(a.out) + ((int64_t)qi * a.H + h) * kD;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = db * 32 + 8 * rr + 4 * g;
          bf16x2 p2 = pack_bf16(o[db][4 * rr] * f, o[db][4 * rr + 1] * f);
          bf16x2 q2 = pack_bf16(o[db][4 * rr + 2] * f, o[db][4 * rr + 3] * f);
          u32x2 w = {__builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, q2)};
          *reinterpret_cast<u32x2 *>(op + d0) = w;
        }
    }
  } else {
    // Part of a pair: O times the head's V scale (so that the combine
    // kernel's merge gives the output directly), m and l into slot 2 p + tail
    // (split) or slot0 + tail (halves), in the layout of the bf16 kernel.
    float *slot = a.part + (int64_t)((wk.slot0 >= 0 ? wk.slot0 : 2 * p) + wk.tail) * kPartFloats;
    const int ql = wave * 32 + col;
    const float vs = a.v_scale[h];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = db * 32 + 8 * rr + 4 * g;
        f32x4 w = {o[db][4 * rr] * vs, o[db][4 * rr + 1] * vs, o[db][4 * rr + 2] * vs,
                   o[db][4 * rr + 3] * vs};
        *reinterpret_cast<f32x4 *>(slot + ql * kD + d0) = w;
      }
    if (g == 0) {
      slot[kBM * kD + ql] = m;
      slot[kBM * kD + kBM + ql] = l;
    }
  }

  // The next item refills the LDS tiles: every wave must be done with
  // this one's.
  lds_barrier();
  }
}

// Quantizing copy of rows [64 c, 64 c + 64) (clipped to T) of one
// compaction job: the K and V rows of window frame sl.src_frame of head
// sl.head go, as e4m3 codes of x / scale, to compacted rows sl.dst_row +
// 64 c ... of k_out / v_out; a thread turns 8 bf16 values (16 bytes) into 8
// e4m3 bytes.
__device__ __forceinline__ void quantize_rows(const WinView &win, int fh_h, CopySlot sl, int cidx,
                                              int T, int D, float sk, float sv, uint8_t *k_out,
                                              uint8_t *v_out) {
  const int r0 = cidx * kCompactRows;
  const int nrows = min(kCompactRows, T - r0);
  const int pieces = D / 8;                 // 16-byte bf16 pieces per row (16)
  const int pieces_shift = __builtin_ctz((unsigned)pieces);
  const int items = nrows * pieces;
  int64_t stride;
  const char *ks = frame_rows(win, false, sl.head, fh_h, sl.src_frame, T, &stride);
  const char *vs = frame_rows(win, true, sl.head, fh_h, sl.src_frame, T, &stride);
  for (int i = threadIdx.x; i < items; i += 256) {
    const int r = i >> pieces_shift, p = i & (pieces - 1);
    const int64_t so = (int64_t)(r0 + r) * stride + p * 16;
    const int64_t d = (sl.dst_row + r0 + r) * (int64_t)D + p * 8;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const u32x4 x = ld16((kv ? vs : ks) + so);
      const float s = kv ? sv : sk;
      u32x2 w;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t lo2 = x[2 * e], hi2 = x[2 * e + 1];
        const float f0 = clamp448(__uint_as_float(lo2 << 16) / s);
        const float f1 = clamp448(__uint_as_float(lo2 & 0xffff0000u) / s);
        const float f2 = clamp448(__uint_as_float(hi2 << 16) / s);
        const float f3 = clamp448(__uint_as_float(hi2 & 0xffff0000u) / s);
        int v = cvt2<false>(f0, f1, 0);
        w[e] = (uint32_t)cvt2<true>(f2, f3, v);
      }
      *reinterpret_cast<u32x2 *>((kv ? v_out : k_out) + d) = w;
    }
  }
}

// Quantizing compaction of the slots the selection wrote: workgroup b
// copies chunk b % chunks of slot b / chunks.
__global__ __launch_bounds__(256) void compact_fp8_kernel(CompactFp8Args a) {
  const int slot = blockIdx.x / a.chunks;
  const int cidx = blockIdx.x - slot * a.chunks;
  const CopySlot sl = a.slots[slot];
  quantize_rows(a.win, a.fh[sl.head], sl, cidx, a.T, a.D, a.k_scale[sl.head],
                a.v_scale[sl.head], a.k_out, a.v_out);
}

// The quantizing copies the plan fixes (static heads' kept frames, every
// head's current chunk; see fixed_slot): workgroup b copies chunk
// b % chunks of job b / chunks.
__global__ __launch_bounds__(256) void compact_fp8_fixed_kernel(FixedCopyPlan p, Fp8Scales sc) {
  const int job = blockIdx.x / p.chunks;
  const int cidx = blockIdx.x - job * p.chunks;
  const CopySlot sl = fixed_slot(p, job);
  quantize_rows(p.win, p.fh[sl.head], sl, cidx, p.T, sc.D, sc.k_scale[sl.head],
                sc.v_scale[sl.head], reinterpret_cast<uint8_t *>(p.k_out),
                reinterpret_cast<uint8_t *>(p.v_out));
}

}  // namespace

hipError_t launch_attend_fp8(const AttendFp8Args &a0, void *part, size_t part_bytes,
                             hipStream_t s) {
  // The bf16 planner and combine kernel serve as they are: same pairs, tiles
  // of 64 keys, two workgroups per CU and partial-result layout.
  AttendArgs c = {};
  c.out = a0.out;
  c.tok_off = a0.tok_off;
  c.n_q = a0.n_q;
  c.H = a0.H;
  c.D = kD;
  const int combine_blocks = plan_attend(c, part, part_bytes);
  AttendFp8Args a = a0;
  a.part = c.part;
  a.n_wg = c.n_wg;
  a.sched = c.sched;
  a.slots_x = c.slots_x;
  a.cut_max = c.cut_max;
  hipLaunchKernelGGL(attend_fp8_kernel, dim3(a.n_wg), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch_attend_combine(c, combine_blocks, s);
  return e;
}

hipError_t launch_compact_fp8_fixed(const FixedCopyPlan &p, const Fp8Scales &sc, hipStream_t s) {
  const int64_t blocks = (int64_t)p.fixed_off_h[p.H] * p.chunks;
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(compact_fp8_fixed_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, sc);
  return hipGetLastError();
}

hipError_t launch_compact_fp8(const CompactFp8Args &a, int total_slots, hipStream_t s) {
  if (total_slots <= 0) return hipSuccess;
  hipLaunchKernelGGL(compact_fp8_kernel, dim3((unsigned)total_slots * (unsigned)a.chunks),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fkv
