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

// v_permlane32_swap with both operands = v: one result holds v of the lower
// half in both halves, the other v of the upper half.  Any symmetric
// combination of the two is the lane-pair (l, l ^ 32) reduction.
__device__ __forceinline__ float pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

}  // namespace fkv
