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

// One workgroup (4 waves) per packed 32-row block, one pass over its input. Lane l of a
// wave owns slot l of the wave's chunks: row l & 31 and the P = 16 / E dimensions of that
// slot, which it loads once (bf16, fp8 and int8 slots hold P consecutive dimensions; an f32
// slot holds every other dimension of 8 consecutive ones, so the lane loads the 8 and keeps
// its 4). The row's sum of squares and max |x| are reduced over the lane pair (l, l ^ 32)
// and the 4 waves in LDS; each lane then converts its values from registers and writes its
// 16-byte slot, so loads and stores are 1 KiB per wave instruction. VEC: src is 16-byte
// aligned and slots are read with 16-byte loads.
template <int DT, int D, bool VEC>
__global__ __launch_bounds__(256) void prepare_kernel(const float* __restrict__ src, int64_t rows,
                                                      int64_t block0, uint8_t* __restrict__ dst,
                                                      float* __restrict__ row_scale) {
  constexpr int NCH = chunks_per_block(DT, D);
  constexpr int CPW = (NCH + 3) / 4;  // chunks per wave: wave w has chunks w*CPW ..
  constexpr int P = DT == MIPS_F32 ? 4 : (DT == MIPS_BF16 ? 8 : 16);
  constexpr int L = DT == MIPS_F32 ? 8 : P;  // floats loaded per slot
  __shared__ float s_ss[4][kFrag];
  __shared__ float s_mx[4][kFrag];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 31;
  const int h = lane >> 5;
  const int64_t blk = blockIdx.x;  // block within this call
  const int64_t lr = blk * kFrag + r;
  const bool live = lr < rows;
  const float* x = src + lr * D;  // read only for live rows

  float v[CPW][P];
  float ss = 0.0f, mx = 0.0f;
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = wave * CPW + i;
    const bool on = live && c < NCH;
    const int base = DT == MIPS_F32 ? 8 * c : slot_dim(DT, c, lane, 0);
    float f[L];
#pragma unroll
    for (int u = 0; u < L; u += 4) {
      if (VEC) {
        const float4 a = on ? *(const float4*)(x + base + u) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        f[u] = a.x;
        f[u + 1] = a.y;
        f[u + 2] = a.z;
        f[u + 3] = a.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[u + e] = on ? x[base + u + e] : 0.0f;
      }
    }
#pragma unroll
    for (int t = 0; t < P; ++t) {
      v[i][t] = DT == MIPS_F32 ? (h ? f[2 * t + 1] : f[2 * t]) : f[t];
      ss = fmaf(v[i][t], v[i][t], ss);
      mx = fmaxf(mx, fabsf(v[i][t]));
    }
  }
  ss += __shfl_xor(ss, 32, kWave);
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  if (lane < kFrag) {
    s_ss[wave][r] = ss;
    s_mx[wave][r] = mx;
  }
  __syncthreads();
  float nrm = 1.0f, amax = 0.0f;
  if (live) {
    nrm = sqrtf(fmaxf((s_ss[0][r] + s_ss[1][r]) + (s_ss[2][r] + s_ss[3][r]), kNormEps));
    // division is monotone, so max |x| / nrm is the max of |x_j| / nrm
    amax = fmaxf(fmaxf(s_mx[0][r], s_mx[1][r]), fmaxf(s_mx[2][r], s_mx[3][r])) / nrm;
  }
  float sdiv = 1.0f;  // int8: the codes are y / scale; fp8: y * 2^-t
  if (DT == MIPS_FP8_E4M3) {
    int t = e4m3_scale_exp(amax);
    t = t < -126 ? -126 : t;
    sdiv = exp2_int(-t);
    if (wave == 0 && lane < kFrag) row_scale[(block0 + blk) * kFrag + r] = exp2_int(t);
  } else if (DT == MIPS_INT8) {
    sdiv = i8_scale(amax);
    if (wave == 0 && lane < kFrag) row_scale[(block0 + blk) * kFrag + r] = sdiv;
  }

  uint8_t* out = dst + (block0 + blk) * block_bytes(DT, D);
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = wave * CPW + i;
    if (c >= NCH) break;
    u32x4_t o = {0u, 0u, 0u, 0u};
    if (DT == MIPS_F32) {
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = __float_as_uint(v[i][t] / nrm);
    } else if (DT == MIPS_BF16) {
#pragma unroll
      for (int t = 0; t < 8; t += 2)
        o[t >> 1] = (uint32_t)f32_to_bf16(v[i][t] / nrm) |
                    ((uint32_t)f32_to_bf16(v[i][t + 1] / nrm) << 16);
    } else if (DT == MIPS_INT8) {
#pragma unroll
      for (int t = 0; t < 16; ++t) o[t >> 2] |= f32_to_i8((v[i][t] / nrm) / sdiv) << (8 * (t & 3));
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t)
        o[t >> 2] |= (uint32_t)f32_to_e4m3((v[i][t] / nrm) * sdiv) << (8 * (t & 3));
    }
    *(u32x4_t*)(out + (int64_t)c * kChunkBytes + lane * 16) = o;
  }
}

template <int DT, int D>
static int launch_prepare(const float* src, int64_t rows, int64_t row_offset, void* dst,
                          float* row_scale, hipStream_t s) {
  const int64_t nblk = (rows + kFrag - 1) / kFrag;
  const bool vec = aligned(src, 16);  // rows are 64-byte multiples: every row stays aligned
  for (int64_t b0 = 0; b0 < nblk; b0 += kMaxGridBlocks) {
    const int64_t nb = nblk - b0 < kMaxGridBlocks ? nblk - b0 : kMaxGridBlocks;
    if (vec)
      hipLaunchKernelGGL((prepare_kernel<DT, D, true>), dim3((unsigned)nb), dim3(256), 0, s,
                         src + b0 * kFrag * D, rows - b0 * kFrag, row_offset / kFrag + b0,
                         (uint8_t*)dst, row_scale);
    else
      hipLaunchKernelGGL((prepare_kernel<DT, D, false>), dim3((unsigned)nb), dim3(256), 0, s,
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
