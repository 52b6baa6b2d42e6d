// Device-side building blocks shared by the gfx950 kernels of libfkv.
//
// MFMA fragment conventions (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand: lane l supplies row (l % 32), k-elements 8*(l/32) .. +7
//   B operand: lane l supplies column (l % 32), k-elements 8*(l/32) .. +7
//   C/D:       lane l holds column (l % 32), rows 8*(r/4) + 4*(l/32) + (r%4)
//              for accumulator registers r = 0..15
// Scores are formed transposed, S^T = K Q^T (rows = keys, columns =
// queries), so that each lane owns one query column: row reductions of the
// softmax stay inside a lane plus one exchange with lane l^32, and the
// accumulator registers of S^T, converted to bf16, are directly the B
// operand of O^T = V^T P^T (with a fixed permutation of the 16 keys of each
// k-step applied identically to V^T).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fkv_launch.h"

namespace fkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// Finite "minus infinity" for running maxima, so that differences of two
// untouched maxima stay 0 instead of NaN.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Exchange with lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float v) {
  return __shfl_xor(v, 32, 64);
}

// v_permlane32_swap / v_permlane16_swap applied to two copies of v (rows are
// 16 lanes, halves 32):
//   permlane32: a = the lower half of v in both halves, b = the upper half;
//   permlane16: a = rows [0, 0, 2, 2] of v, b = rows [1, 1, 3, 3].
// Written in inline assembly: given the same value twice, the compiler's
// builtin may fold its two results into one (seen with ROCm 7.2), which is
// wrong for these cross-lane swaps.  The s_nop gives the two wait states that
// a VALU write of the source registers needs before the swap reads them.
struct LanePair {
  uint32_t a, b;
};
__device__ __forceinline__ LanePair permlane32_swap_copies(uint32_t v) {
  uint32_t a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return LanePair{a, b};
}
__device__ __forceinline__ LanePair permlane16_swap_copies(uint32_t v) {
  uint32_t a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return LanePair{a, b};
}

// Lane-pair (l, l ^ 32) reductions: any symmetric combination of the two
// halves of a permlane32 swap.
__device__ __forceinline__ float pair_max(float v) {
  const LanePair r = permlane32_swap_copies(__float_as_uint(v));
  return fmaxf(__uint_as_float(r.a), __uint_as_float(r.b));
}
__device__ __forceinline__ float pair_sum(float v) {
  const LanePair r = permlane32_swap_copies(__float_as_uint(v));
  return __uint_as_float(r.a) + __uint_as_float(r.b);
}

// s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt left at their maxima):
// waits until this wave's vector-memory loads, including loads that write
// LDS directly, have completed.
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for code that moves data into LDS only through
// buffer loads with the LDS destination (whose completion the caller waits
// for explicitly with s_waitcnt vmcnt): waits for this wave's own LDS reads and writes
// (lgkmcnt(0)), then s_barrier.  Unlike __syncthreads() it carries no
// memory fence, so copies still in flight for later tiles are not waited
// for.  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer resource over `bytes` bytes starting at `base` (raw addressing,
// stride 0).  Loads at offsets past the end return zeros; word 3 = 0x00020000
// is the gfx9 data-format setting for untyped dword loads.
// The base and size must be wave-uniform; they are passed through
// readfirstlane so that the compiler keeps the descriptor in scalar registers
// (a descriptor it believes divergent costs a loop over lanes per load).
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void *base, uint32_t bytes) {
  // readfirstlane returns int: go through uint32_t so neither half is
  // sign-extended when the 64-bit address is put back together.
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint64_t up = ((uint64_t)hi << 32) | (uint64_t)lo;
  const int ub = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(up), (short)0, ub,
                                           0x00020000);
}

// 16-byte buffer -> LDS copy (buffer_load_dwordx4 ... lds): lane i's 16 bytes
// at rsrc + soffset + voffset + IMM land at lds_wave_base + IMM + 16 i (the
// instruction's immediate offset applies to both addresses).  lds_wave_base
// must be wave-uniform and 1 KiB aligned.  Out-of-range lanes write zeros.
// Several copies sharing one LDS base and differing by IMM need one M0 value.
template <int IMM = 0>
__device__ __forceinline__ void buffer_load_lds16(buf_rsrc rsrc, uint32_t voffset,
                                                  uint32_t soffset, void *lds_wave_base) {
  static_assert(IMM >= 0 && IMM < 4096, "12-bit immediate offset");
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void *)lds_wave_base, 16, voffset, soffset, IMM,
      0);
}

// Four 16-byte copies into 4 consecutive KiB of LDS (one wave's 16 tile
// rows): voff[j] already has j KiB subtracted, so the immediate offsets
// 0, 1, 2, 3 KiB restore the global address and place the LDS rows.
__device__ __forceinline__ void buffer_load_lds16x4(buf_rsrc rsrc, const uint32_t *voff,
                                                    uint32_t soffset, void *lds_wave_base) {
  buffer_load_lds16<0>(rsrc, voff[0], soffset, lds_wave_base);
  buffer_load_lds16<1024>(rsrc, voff[1], soffset, lds_wave_base);
  buffer_load_lds16<2048>(rsrc, voff[2], soffset, lds_wave_base);
  buffer_load_lds16<3072>(rsrc, voff[3], soffset, lds_wave_base);
}

__device__ __forceinline__ bf16x2 pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);
}

// ---------------------------------------------------------------------------
// K / V tiles in LDS: KT rows (keys) x 128 bf16 (256 B per row), row-major.
// The 16-byte chunk c of row j sits at chunk position c ^ swz(j) with
// swz(j) = ((j & 3) << 2) | ((j >> 2) & 3).  With 64 banks of 4 bytes this
// keeps the three access patterns of the tile free of bank conflicts:
//   - 16 lanes writing the 16 chunks of one row;
//   - 16 lanes reading 16 consecutive rows at one chunk (ds_read_b128, the
//     K fragments of S^T): swz is a permutation of 0..15 over any aligned
//     16 rows;
//   - 32 lanes of a transposing read (ds_read_b64_tr_b16, the V^T
//     fragments) covering 4 aligned consecutive rows x an aligned group of 4
//     chunks: bits 2-3 of swz take the 4 values over those rows, so the 4
//     rows' chunk groups fall on disjoint banks.
template <int KT>
struct KvTileLds {
  static constexpr int kBytes = KT * 256;
  __device__ static __forceinline__ uint32_t swz(int row) {
    return (uint32_t)(((row & 3) << 2) | ((row >> 2) & 3));
  }
  __device__ static __forceinline__ uint32_t offset(int row, int chunk) {
    return (uint32_t)(row * 256) + (((uint32_t)chunk ^ swz(row)) << 4);
  }
};

// Transposing LDS read (ds_read_b64_tr_b16, gfx950).  Within each group of 16
// lanes, lane s = 4 j + c supplies the address of 4 consecutive 16-bit
// elements of row k0 + j at columns n0 + 4 c .. n0 + 4 c + 3; lane i of the
// group receives column n0 + i of rows k0 .. k0 + 3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const char *base, uint32_t off) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  lds_s16x4 *p = (lds_s16x4 *)(base + off);  // generic -> LDS address space
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
}

__device__ __forceinline__ u32x4 lds_read_b128(const char *base, uint32_t off) {
  return *reinterpret_cast<const u32x4 *>(base + off);
}

// Global 16-byte load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
// Streaming forms (non-temporal hint): data touched once, kept from
// displacing lines that other workgroups re-read from L2.
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void st16_stream(void *p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// First byte of the T-row frame f of head h's window (fh_h history frames,
// then the current chunk; see WinView), and the bytes between its rows.
__device__ __forceinline__ const char *frame_rows(const WinView &w, bool want_v, int h, int fh_h,
                                                  int f, int T, int64_t *row_stride) {
  if (f < fh_h) {
    const char *base = want_v ? w.hist_v : w.hist_k;
    if (w.hist_off) {
      *row_stride = w.row_bytes;
      return base + (w.hist_off[h] + (int64_t)f * T) * w.row_bytes;
    }
    *row_stride = w.tm_row_bytes;
    return base + (int64_t)f * T * w.tm_row_bytes + (int64_t)h * w.row_bytes;
  }
  const char *base = want_v ? w.cur_v : w.cur_k;
  *row_stride = w.tm_row_bytes;
  return base + (int64_t)(f - fh_h) * T * w.tm_row_bytes + (int64_t)h * w.row_bytes;
}

// Copy of rows [64 c, 64 c + 64) (clipped to T) of one compaction job: the
// K and V rows of window frame sl.src_frame of head sl.head go to compacted
// rows sl.dst_row + 64 c ... of k_out / v_out.  256 threads, 16-byte pieces,
// eight loads in flight per thread before the stores.
__device__ __forceinline__ void copy_rows(const WinView &win, int fh_h, CopySlot sl, int c,
                                          int T, char *k_out, char *v_out) {
  constexpr int kThreads = 256;
  const int r0 = c * kCompactRows;
  const int nrows = min(kCompactRows, T - r0);
  const int row_bytes = win.row_bytes;
  const int v16 = row_bytes >> 4;          // 16-byte pieces per row
  // rows are 128, 256 or 512 bytes (D of 64 or 128, bf16 or fp32): a power
  // of two, so row and piece come from a shift and a mask
  const int v16_shift = __builtin_ctz((unsigned)v16);
  const int items = nrows * v16;
  int64_t src_stride;
  const char *ks = frame_rows(win, false, sl.head, fh_h, sl.src_frame, T, &src_stride) +
                   r0 * src_stride;
  const char *vs = frame_rows(win, true, sl.head, fh_h, sl.src_frame, T, &src_stride) +
                   r0 * src_stride;
  char *kd = k_out + (sl.dst_row + r0) * row_bytes;
  char *vd = v_out + (sl.dst_row + r0) * row_bytes;
  constexpr int U = 4;
  for (int base = 0; base < items; base += kThreads * U) {
    u32x4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * kThreads + threadIdx.x;
      if (idx < items) {
        const int r = idx >> v16_shift, p = idx & (v16 - 1);
        const int64_t so = r * src_stride + p * 16;
        kr[u] = ld16_stream(ks + so);
        vr[u] = ld16_stream(vs + so);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * kThreads + threadIdx.x;
      if (idx < items) {
        st16_stream(kd + (int64_t)idx * 16, kr[u]);
        st16_stream(vd + (int64_t)idx * 16, vr[u]);
      }
    }
  }
}

// The data-independent compaction job s (0 <= s < p.fixed_off_h[H]): the
// kept history frames of static heads and the current-chunk frames of every
// head, which the host plan fixes before any score is known.  Head h owns
// jobs [fixed_off_h[h], fixed_off_h[h+1]): first its n_hist_fixed[h] kept
// history frames (the set bits of static_bits[h], ascending; 0 for dynamic
// heads), then its F_c current frames, which follow the head's kept[h]
// history frames in its compacted range.
__device__ __forceinline__ CopySlot fixed_slot(const FixedCopyPlan &p, int s) {
  int h = 0;
  while (h + 1 < p.H && p.fixed_off_h[h + 1] <= s) ++h;
  const int j = s - p.fixed_off_h[h];
  CopySlot sl;
  sl.head = h;
  if (j < p.n_hist_fixed[h]) {
    uint64_t b = p.static_bits[h];
    for (int i = 0; i < j; ++i) b &= b - 1ull;
    sl.src_frame = __ffsll((long long)b) - 1;
    sl.dst_row = p.tok_off_h[h] + (int64_t)j * p.T;
  } else {
    const int cf = j - p.n_hist_fixed[h];
    sl.src_frame = p.fh[h] + cf;
    sl.dst_row = p.tok_off_h[h] + (int64_t)(p.kept[h] + cf) * p.T;
  }
  return sl;
}

// ---- attention schedules (bf16 and fp8 kernels, and their launchers) ----
//
// Split schedule on XCD x (nb workgroups, nb % 8 == 0, at most nb / 2
// pairs): the XCD's pairs are [p_lo, p_lo + np) and its workgroups
// xs = 0 .. nb/8 - 1.  The first np workgroups run tiles [0, split) of one
// pair each (main parts), the ne others the tails [split, tiles) of up to
// k = ceil(np / ne) pairs each (k = 0: no cut).
struct XcdSplit {
  int p_lo, np, ne, k;
};
__host__ __device__ __forceinline__ XcdSplit xcd_split(int pairs, int nb, int x) {
  XcdSplit s;
  s.p_lo = pairs * x / 8;
  s.np = pairs * (x + 1) / 8 - s.p_lo;
  s.ne = nb / 8 - s.np;
  s.k = s.ne > 0 ? (s.np + s.ne - 1) / s.ne : 0;
  return s;
}
// Rounds schedule on XCD x (more pairs than resident workgroups): the XCD's
// pairs are [p_lo, p_lo + np) and slots_x workgroups of it run at a time.
// The first w pairs run whole, one workgroup each, in full rounds plus part
// of the last; the s pairs after them are cut in two halves (tiles
// [0, nt/2) and [nt/2, nt)) so that the last round is full too: with
// rem = np mod slots_x, s = rem when 2 rem <= slots_x (the last round is
// halves only), else s = slots_x - rem (rem - s whole pairs and 2 s halves).
struct XcdRounds {
  int p_lo, np, w, s;
};
__host__ __device__ __forceinline__ XcdRounds xcd_rounds(int pairs, int slots_x, int x) {
  XcdRounds r;
  r.p_lo = pairs * x / 8;
  r.np = pairs * (x + 1) / 8 - r.p_lo;
  const int rem = r.np % slots_x;
  r.s = rem == 0 ? 0 : (2 * rem <= slots_x ? rem : slots_x - rem);
  r.w = r.np - r.s;
  return r;
}

// First tail tile of a pair with nt tiles (nt when nothing is cut).  A
// tail workgroup runs its k tails one after the other, each restarting the
// copy pipeline, and takes about 9/8 the time per tile of a main workgroup;
// split = nt * 9k / (8 + 9k) evens out the two.
__host__ __device__ __forceinline__ int split_tile(int nt, int k) {
  return k > 0 ? (int)((int64_t)nt * (9 * k) / (8 + 9 * k)) : nt;
}

// What one workgroup of an attention launch does: n_items pairs p0, p0 + 1,
// ... (tail parts of the split schedule: one each), cut as k says (0: whole
// pairs, > 0: split_tile(nt, k), -1: halves), the tail part when tail is 1,
// partial results in slot0 (halves) or 2 p + tail (split).  n_items < 0:
// nothing (padding of the rounds schedule).  Without a partial-result
// buffer every workgroup takes one whole pair, each XCD (workgroup b runs on
// XCD b % 8) a contiguous run of them.
struct AttendWork {
  int p0, n_items, k, tail, slot0;
};
__device__ __forceinline__ AttendWork attend_work(int pairs, bool has_part, int sched,
                                                  int slots_x, int cut_max, int nb, int b) {
  const int x = b & 7, xs = b >> 3;
  AttendWork w;
  w.k = 0;
  w.tail = 0;
  w.slot0 = -1;
  w.n_items = 1;
  if (!has_part) {
    w.p0 = x * (nb >> 3) + min(x, nb & 7) + xs;
  } else if (sched == 2) {
    const XcdRounds xr = xcd_rounds(pairs, slots_x, x);
    if (xs < xr.w) {
      w.p0 = xr.p_lo + xs;
    } else if (xs < xr.w + 2 * xr.s) {
      const int c = (xs - xr.w) >> 1;
      w.tail = (xs - xr.w) & 1;
      w.p0 = xr.p_lo + xr.w + c;
      w.k = -1;  // halves
      w.slot0 = 2 * (x * cut_max + c);
    } else {
      w.p0 = 0;
      w.n_items = -1;
    }
  } else {
    const XcdSplit sp = xcd_split(pairs, nb, x);
    w.k = sp.k;
    if (xs < sp.np) {
      w.p0 = sp.p_lo + xs;
    } else {
      const int e = xs - sp.np;
      w.p0 = sp.p_lo + e * sp.np / sp.ne;
      w.n_items = sp.p_lo + (e + 1) * sp.np / sp.ne - w.p0;
      w.tail = 1;
    }
  }
  return w;
}

}  // namespace fkv
