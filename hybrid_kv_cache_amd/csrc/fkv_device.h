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

__device__ __forceinline__ bf16x2 pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);
}

// ---------------------------------------------------------------------------
// K tile in LDS: KT rows (keys) x 128 bf16 (256 B); the 16-byte chunk c of row
// j is stored at chunk position c ^ (j & 15), so that 16 consecutive rows read
// at one chunk column hit 16 distinct bank groups.
template <int KT>
struct KTileLds {
  static constexpr int kBytes = KT * 256;
  __device__ static __forceinline__ uint32_t offset(int row, int chunk) {
    return (uint32_t)(row * 256 + ((chunk ^ (row & 15)) << 4));
  }
};

// V^T tile in LDS: 128 rows (head dim) x KT keys bf16.  Keys are grouped in
// 8-byte groups of 4; group G of row d sits at position G ^ swz(d) with
// swz(d) = (d + (d >> 4)) & 15, spreading both the transposing writes (16
// rows of one key group) and the fragment reads (32 rows of one key group)
// over distinct banks.  KT must be 64 (16 groups per row).
struct VtTileLds {
  static constexpr int KT = 64;
  static constexpr int kRowBytes = KT * 2;
  static constexpr int kBytes = 128 * kRowBytes;
  __device__ static __forceinline__ uint32_t offset(int d, int group) {
    int swz = (d + (d >> 4)) & 15;
    return (uint32_t)(d * kRowBytes + ((group ^ swz) << 3));
  }
};

__device__ __forceinline__ u32x4 lds_read_b128(const char *base, uint32_t off) {
  return *reinterpret_cast<const u32x4 *>(base + off);
}
__device__ __forceinline__ u32x2 lds_read_b64(const char *base, uint32_t off) {
  return *reinterpret_cast<const u32x2 *>(base + off);
}

// Global 16-byte load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// Pair two 16-bit halves into one dword: (lo16(a), lo16(b)) or (hi16(a), hi16(b)).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

}  // namespace fkv
