// normalize.hip -- row L2 normalisation and the packed-corpus build for gfx950.
//
// y = x / sqrt(max(sum x^2, 1e-12)) per row: the form of `_l2_normalize_candidates`
// and of the user-representation normalisation in recsys_two_tower_model.py
// (x-algorithm Phoenix). HBM-bound: every kernel reads each input element once and
// writes each output element once.
#include "common.h"
#include "host.h"

namespace mips {

constexpr float kNormEps = 1e-12f;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// One wave per row. Lane j sums dims j, j+64, ...; the butterfly fixes the order.
template <int OUT>
__global__ __launch_bounds__(256) void l2_normalize_kernel(const float* __restrict__ src,
                                                           int64_t rows, int d,
                                                           void* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* x = src + row * d;
  float ss = 0.0f;
  for (int j = lane; j < d; j += kWave) ss = fmaf(x[j], x[j], ss);
  ss = wave_sum(ss);
  const float nrm = sqrtf(fmaxf(ss, kNormEps));
  for (int j = lane; j < d; j += kWave) {
    const float y = x[j] / nrm;
    if (OUT == MIPS_F32)
      ((float*)dst)[row * d + j] = y;
    else
      ((uint16_t*)dst)[row * d + j] = f32_to_bf16(y);
  }
}

// One workgroup (4 waves) per packed 32-row block. Phase 1: each wave normalises 8
// rows' norms (and, for E4M3, the row's power-of-two scale; for int8, max|y| / 127). Phase 2: the block's
// 1 KiB chunks are written, one 16-byte slot per lane, so stores are fully coalesced.
template <int DT, int D>
__global__ __launch_bounds__(256) void prepare_kernel(const float* __restrict__ src, int64_t rows,
                                                      int64_t block0, uint8_t* __restrict__ dst,
                                                      float* __restrict__ row_scale) {
  constexpr int NCH = chunks_per_block(DT, D);
  __shared__ float s_norm[kFrag];
  __shared__ float s_scale_inv[kFrag];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t blk = blockIdx.x;             // block within this call
  const int64_t row_base = blk * kFrag;       // local row of the block's first row

  for (int r = wave; r < kFrag; r += 4) {
    const int64_t lr = row_base + r;
    float nrm = 1.0f, amax = 0.0f;
    if (lr < rows) {
      const float* x = src + lr * D;
      float ss = 0.0f;
      for (int j = lane; j < D; j += kWave) ss = fmaf(x[j], x[j], ss);
      ss = wave_sum(ss);
      nrm = sqrtf(fmaxf(ss, kNormEps));
      if (DT == MIPS_FP8_E4M3 || DT == MIPS_INT8) {
        float m = 0.0f;
        for (int j = lane; j < D; j += kWave) m = fmaxf(m, fabsf(x[j] / nrm));
        amax = wave_max(m);
      }
    }
    if (lane == 0) {
      s_norm[r] = nrm;
      if (DT == MIPS_FP8_E4M3) {
        int t = e4m3_scale_exp(amax);
        t = t < -126 ? -126 : t;
        s_scale_inv[r] = exp2_int(-t);
        row_scale[(block0 + blk) * kFrag + r] = exp2_int(t);
      } else if (DT == MIPS_INT8) {
        const float sc = i8_scale(amax);
        s_scale_inv[r] = sc;  // int8 divides by the scale itself
        row_scale[(block0 + blk) * kFrag + r] = sc;
      }
    }
  }
  __syncthreads();

  uint8_t* out = dst + (block0 + blk) * block_bytes(DT, D);
  for (int c = wave; c < NCH; c += 4) {
    const int r = lane & 31;
    const int64_t lr = row_base + r;
    const bool live = lr < rows;
    const float* x = src + lr * D;
    const float nrm = s_norm[r];
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (DT == MIPS_F32) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float y = live ? x[slot_dim(DT, c, lane, t)] / nrm : 0.0f;
        v[t] = __float_as_uint(y);
      }
    } else if (DT == MIPS_BF16) {
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        const float y0 = live ? x[slot_dim(DT, c, lane, t)] / nrm : 0.0f;
        const float y1 = live ? x[slot_dim(DT, c, lane, t + 1)] / nrm : 0.0f;
        v[t >> 1] = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
      }
    } else if (DT == MIPS_INT8) {
      const float sc = s_scale_inv[r];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float y = live ? (x[slot_dim(DT, c, lane, t)] / nrm) / sc : 0.0f;
        v[t >> 2] |= f32_to_i8(y) << (8 * (t & 3));
      }
    } else {
      const float sinv = s_scale_inv[r];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float y = live ? (x[slot_dim(DT, c, lane, t)] / nrm) * sinv : 0.0f;
        v[t >> 2] |= (uint32_t)f32_to_e4m3(y) << (8 * (t & 3));
      }
    }
    *(u32x4_t*)(out + (int64_t)c * kChunkBytes + lane * 16) = v;
  }
}

template <int DT, int D>
static int launch_prepare(const float* src, int64_t rows, int64_t row_offset, void* dst,
                          float* row_scale, hipStream_t s) {
  const int64_t nblk = (rows + kFrag - 1) / kFrag;
  for (int64_t b0 = 0; b0 < nblk; b0 += kMaxGridBlocks) {
    const int64_t nb = nblk - b0 < kMaxGridBlocks ? nblk - b0 : kMaxGridBlocks;
    hipLaunchKernelGGL((prepare_kernel<DT, D>), dim3((unsigned)nb), dim3(256), 0, s,
                       src + b0 * kFrag * D, rows - b0 * kFrag, row_offset / kFrag + b0,
                       (uint8_t*)dst, row_scale);
    if (const int rc = check_launch()) return rc;
  }
  return MIPS_OK;
}

template <int DT>
static int dispatch_prepare_d(const float* src, int64_t rows, int64_t row_offset, int d,
                              void* dst, float* row_scale, hipStream_t s) {
  switch (d) {
    case 16: if constexpr (DT != MIPS_FP8_E4M3 && DT != MIPS_INT8) return launch_prepare<DT, 16>(src, rows, row_offset, dst, row_scale, s); break;
    case 32: if constexpr (DT != MIPS_FP8_E4M3) return launch_prepare<DT, 32>(src, rows, row_offset, dst, row_scale, s); break;
    case 64: return launch_prepare<DT, 64>(src, rows, row_offset, dst, row_scale, s);
    case 128: return launch_prepare<DT, 128>(src, rows, row_offset, dst, row_scale, s);
    case 256: if constexpr (DT != MIPS_F32) return launch_prepare<DT, 256>(src, rows, row_offset, dst, row_scale, s); break;
  }
  return MIPS_ERR_UNSUPPORTED;
}

}  // namespace mips

extern "C" {

int64_t mips_corpus_bytes(int64_t n, int32_t d, int32_t dtype) {
  if (n < 1 || !mips::corpus_d_supported(dtype, d)) return -1;
  return ((n + 31) / 32) * mips::block_bytes(dtype, d);
}

int64_t mips_scale_count(int64_t n) { return n < 1 ? 0 : ((n + 31) / 32) * 32; }

int mips_l2_normalize(const float* src, int64_t rows, int32_t d, int32_t out_dtype, void* dst,
                      void* stream) {
  if (!src || !dst || rows < 0 || d < 1 || d > 4096) return MIPS_ERR_INVALID_ARG;
  if (out_dtype != MIPS_F32 && out_dtype != MIPS_BF16) return MIPS_ERR_UNSUPPORTED;
  if (!mips::aligned(src, 4) || !mips::aligned(dst, out_dtype == MIPS_F32 ? 4 : 2))
    return MIPS_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  // four rows per workgroup, in launches of at most kMaxGridBlocks workgroups
  const int64_t per = mips::kMaxGridBlocks * 4;
  for (int64_t r0 = 0; r0 < rows; r0 += per) {
    const int64_t nr = rows - r0 < per ? rows - r0 : per;
    const dim3 grid((unsigned)((nr + 3) / 4));
    if (out_dtype == MIPS_F32)
      hipLaunchKernelGGL(mips::l2_normalize_kernel<MIPS_F32>, grid, dim3(256), 0, s, src + r0 * d,
                         nr, d, (void*)((float*)dst + r0 * d));
    else
      hipLaunchKernelGGL(mips::l2_normalize_kernel<MIPS_BF16>, grid, dim3(256), 0, s,
                         src + r0 * d, nr, d, (void*)((uint16_t*)dst + r0 * d));
    if (const int rc = mips::check_launch()) return rc;
  }
  return MIPS_OK;
}

int mips_prepare_corpus(const float* src, int64_t rows, int64_t row_offset, int32_t d,
                        int32_t dtype, void* dst, float* row_scale, void* stream) {
  if (!src || !dst || rows < 1 || row_offset < 0 || (row_offset % 32) != 0)
    return MIPS_ERR_INVALID_ARG;
  if (dtype != MIPS_F32 && dtype != MIPS_BF16 && dtype != MIPS_FP8_E4M3 && dtype != MIPS_INT8)
    return MIPS_ERR_UNSUPPORTED;
  if (!mips::corpus_d_supported(dtype, d)) return MIPS_ERR_UNSUPPORTED;
  if ((dtype == MIPS_FP8_E4M3 || dtype == MIPS_INT8) && !row_scale) return MIPS_ERR_INVALID_ARG;
  if (!mips::aligned(src, 4) || !mips::aligned(dst, 16) ||
      (row_scale && !mips::aligned(row_scale, 4)))
    return MIPS_ERR_INVALID_ARG;
  if ((rows + 31) / 32 > 0x7FFFFFFF) return MIPS_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  switch (dtype) {
    case MIPS_F32:
      return mips::dispatch_prepare_d<MIPS_F32>(src, rows, row_offset, d, dst, row_scale, s);
    case MIPS_BF16:
      return mips::dispatch_prepare_d<MIPS_BF16>(src, rows, row_offset, d, dst, row_scale, s);
    case MIPS_INT8:
      return mips::dispatch_prepare_d<MIPS_INT8>(src, rows, row_offset, d, dst, row_scale, s);
    default:
      return mips::dispatch_prepare_d<MIPS_FP8_E4M3>(src, rows, row_offset, d, dst, row_scale, s);
  }
}

}  // extern "C"
