// common.h -- device helpers shared by the gfx950 kernels of libmips.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mips.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace mips {

constexpr int kWave = 64;
constexpr int kFrag = 32;          // rows per packed block = MFMA M/N
constexpr int kChunkBytes = 1024;  // one wave-wide 16-byte-per-lane load

__host__ __device__ constexpr int elem_bytes(int dtype) {
  return dtype == MIPS_F32 ? 4 : (dtype == MIPS_BF16 ? 2 : 1);
}
// 1 KiB chunks per 32-row block.
__host__ __device__ constexpr int chunks_per_block(int dtype, int d) {
  return d * elem_bytes(dtype) * kFrag / kChunkBytes;
}
__host__ __device__ constexpr int64_t block_bytes(int dtype, int d) {
  return (int64_t)d * elem_bytes(dtype) * kFrag;
}

// Dimension held by element t of slot s (lane) in chunk c of a packed block.
__host__ __device__ inline int slot_dim(int dtype, int c, int s, int t) {
  const int h = s >> 5;
  if (dtype == MIPS_F32) return 8 * c + 2 * t + h;
  if (dtype == MIPS_BF16) return 16 * c + 8 * h + t;
  if (dtype == MIPS_INT8) return 32 * c + 16 * h + t;
  return 64 * (c >> 1) + 32 * h + 16 * (c & 1) + t;
}

// Byte offset of element (row, dim) of a packed matrix.
__host__ __device__ inline int64_t packed_offset(int dtype, int d, int64_t row, int dim) {
  const int E = elem_bytes(dtype);
  int c, h, t;
  if (dtype == MIPS_F32) {
    c = dim >> 3;
    h = dim & 1;
    t = (dim & 7) >> 1;
  } else if (dtype == MIPS_BF16) {
    c = dim >> 4;
    h = (dim >> 3) & 1;
    t = dim & 7;
  } else if (dtype == MIPS_INT8) {
    c = dim >> 5;
    h = (dim >> 4) & 1;
    t = dim & 15;
  } else {
    const int w = dim & 63;
    c = 2 * (dim >> 6) + ((w >> 4) & 1);
    h = w >> 5;
    t = w & 15;
  }
  const int s = (int)(row & 31) + 32 * h;
  return (row >> 5) * block_bytes(dtype, d) + (int64_t)c * kChunkBytes + s * 16 + t * E;
}

// ------------------------------------------------------------ order-preserving keys
// Larger key <=> larger score; -0.0 maps to the key of +0.0. Key 0 is below every
// finite score and means "no threshold".
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
// Threshold key -> float for a `score >= thr` test.
__device__ __forceinline__ float key_threshold(uint32_t k) {
  return k == 0u ? -INFINITY : key_score(k);
}
// Composite key: score descending, then id ascending.
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t id) {
  return ((uint64_t)key << 32) | (uint32_t)(~id);
}
__device__ __forceinline__ uint32_t composite_id(uint64_t c) { return ~(uint32_t)c; }

// ---------------------------------------------------------------- conversions
// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> OCP E4M3 code, round to nearest even, saturating at +-448. The mantissa is
// rounded on the bit pattern: keep 3 of the 23 fraction bits.
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a >= 448.0f) return (uint8_t)(sign | 0x7Eu);
  if (a < 0.015625f) {  // below 2^-6: subnormal codes, step 2^-9
    const int m = (int)rintf(a * 512.0f);
    return (uint8_t)(sign | (uint32_t)m);
  }
  const uint32_t ua = __float_as_uint(a);
  int e = (int)(ua >> 23) - 127;
  const uint32_t frac = ua & 0x7FFFFFu;
  uint32_t keep = frac >> 20;
  const uint32_t rest = frac & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) {
    keep = 0u;
    ++e;
  }
  return (uint8_t)(sign | ((uint32_t)(e + 7) << 3) | keep);
}
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = (e == 0u) ? (float)m * 0.001953125f  // m * 2^-9
                      : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -v : v;
}

// Exponent t of the power-of-two scale 2^t: the smallest t with amax <= 448 * 2^t
// (t = 0 for amax == 0). amax = f * 2^e with f in [0.5, 1) from the bit pattern.
__device__ __forceinline__ int e4m3_scale_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const uint32_t u = __float_as_uint(amax);
  const int e = (int)(u >> 23) - 126;                 // amax = f * 2^e, f in [0.5, 1)
  const uint32_t frac = u & 0x7FFFFFu;                // f = (1 + frac/2^23) / 2
  return (frac <= 0x600000u) ? e - 9 : e - 8;         // f <= 0.875 <=> frac <= 0.75 * 2^23
}

// int8 codes with one float scale per row: scale = max(amax / 127, 1e-12), code =
// nearest integer to v / scale (ties to even), clipped to [-127, 127].
__device__ __forceinline__ float i8_scale(float amax) { return fmaxf(amax / 127.0f, 1e-12f); }
__device__ __forceinline__ uint32_t f32_to_i8(float v) {
  const float r = fminf(fmaxf(rintf(v), -127.0f), 127.0f);
  return (uint32_t)(int)r & 0xFFu;
}

__device__ __forceinline__ float exp2_int(int t) {  // 2^t for |t| <= 126
  return __uint_as_float((uint32_t)(t + 127) << 23);
}

// -------------------------------------------------------------- MFMA output map
// Row of the 32x32 tile held by accumulator register i of lane `lane`; the column is
// lane & 31 (v_mfma_f32_32x32x* output layout).
__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

}  // namespace mips
