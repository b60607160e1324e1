// topk.hip -- exhaustive inner-product top-K for gfx950 (MI355X).
//
// The serving step of two-tower retrieval: score a batch of normalised user vectors
// against the whole normalised index by dot product and keep each user's K best
// (`RecsysTwoTowerModel.forward` in recsys_two_tower_model.py; Phoenix README, "How
// Retrieval Works", step 4). The score matrix is never written out. One call runs:
//
//   prep_queries     queries -> MFMA operand layout (E4M3 + power-of-two scale for an
//                    fp8 corpus); clears the per-query state.
//   score<SAMPLE>    (large N only) scores a prefix sample of the corpus and writes
//                    per-(query, 32-row block) maxima: "delegates".
//   sample_threshold per query, the K-th largest delegate: K distinct blocks hold an
//                    item at least that good, so it is a lower bound of the K-th best
//                    score (the starting threshold), plus a few higher "levels".
//   score<MAIN>      streams the packed corpus HBM -> VGPR (1 KiB coalesced wave loads)
//                    against the query block staged in LDS, on the 32x32 MFMA, and
//                    keeps in registers only a per-lane max; blocks whose max clears the
//                    query's threshold are re-checked item by item (exclusion bitmap,
//                    threshold) and survivors are appended to the query's candidate
//                    list. Counting survivors above each level raises the threshold
//                    (atomicMax) once K of them exist.
//   final_select     per query, a radix select over the 64-bit composite keys
//                    (score key << 32 | ~id) of its candidates, then a bitonic sort:
//                    score descending, then id ascending. A query whose list overflowed
//                    is rescanned exactly by its workgroup.
#include <algorithm>

#include "common.h"
#include "host.h"

namespace mips {

constexpr int kLevels = 8;          // threshold levels per query
constexpr int kScoreThreads = 512;  // 8 waves
constexpr int kScoreWaves = kScoreThreads / kWave;
constexpr int kSampleGroups = 8192; // delegates per query (prefix sample of 8192 blocks)
constexpr int kSelThreads = 256;
constexpr int kFallbackBuf = 4096;  // fallback candidate buffer (entries)
constexpr int kLdsScoreBudget = 150 * 1024;  // query block + scales + per-wave thresholds

// Fragments (32-row blocks) per wave tile: keeps the corpus operand at <= 128 VGPRs
// (a fragment's operand is d * elem_bytes / 8 VGPRs per lane).
__host__ __device__ constexpr int tile_frags(int ct, int d) {
  const int r = 1024 / (d * elem_bytes(ct));
  return r < 1 ? 1 : (r > 8 ? 8 : r);
}

enum { MODE_SAMPLE = 0, MODE_MAIN = 1 };

struct ScoreArgs {
  const uint8_t* corpus;
  const float* row_scale;
  const uint32_t* exclude;
  const uint8_t* qtile;
  const int* qexp;
  int64_t n;
  int64_t n32;      // 32-row blocks in the corpus
  int64_t nfrag;    // blocks this pass covers (n32, or the sample size)
  int64_t ntiles;   // wave tiles this pass covers
  int b;
  int b32;
  int qb;           // queries per query block
  int nqblk;
  int nslices;
  int k;
  int64_t cap;
  uint32_t* thr;
  const uint32_t* lvl;
  uint32_t* lcnt;
  uint32_t* cnt;
  uint64_t* cand;
  uint32_t* delegates;
  int G;
};

__device__ __forceinline__ float neg_inf() { return -INFINITY; }

template <int CT>
__device__ __forceinline__ void mfma_step(f32x16_t& acc, const u32x4_t* a, const u32x4_t* b,
                                          int sa, int sb, int s) {
  if constexpr (CT == MIPS_BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[s]),
                                                  __builtin_bit_cast(bf16x8_t, b[s]), acc, 0, 0, 0);
  } else if constexpr (CT == MIPS_FP8_E4M3) {
    i32x8_t av, bv;
    av[0] = (int)a[2 * s][0]; av[1] = (int)a[2 * s][1]; av[2] = (int)a[2 * s][2]; av[3] = (int)a[2 * s][3];
    av[4] = (int)a[2 * s + 1][0]; av[5] = (int)a[2 * s + 1][1]; av[6] = (int)a[2 * s + 1][2]; av[7] = (int)a[2 * s + 1][3];
    bv[0] = (int)b[2 * s][0]; bv[1] = (int)b[2 * s][1]; bv[2] = (int)b[2 * s][2]; bv[3] = (int)b[2 * s][3];
    bv[4] = (int)b[2 * s + 1][0]; bv[5] = (int)b[2 * s + 1][1]; bv[6] = (int)b[2 * s + 1][2]; bv[7] = (int)b[2 * s + 1][3];
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, sa, 0, sb);
  } else {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[s >> 2][s & 3]),
                                               __uint_as_float(b[s >> 2][s & 3]), acc, 0, 0, 0);
  }
}

// Appends one survivor of query q and counts it against the query's levels.
__device__ __forceinline__ void append_candidate(const ScoreArgs& A, int q, float v, uint32_t id) {
  const uint32_t key = score_key(v);
  const uint32_t pos = atomicAdd(&A.cnt[q], 1u);
  if ((int64_t)pos < A.cap) A.cand[(int64_t)q * A.cap + pos] = composite(key, id);
  const uint32_t* L = A.lvl + (int64_t)q * kLevels;
  uint32_t* C = A.lcnt + (int64_t)q * kLevels;
#pragma unroll
  for (int j = 0; j < kLevels; ++j) {
    const uint32_t lj = L[j];
    if (key >= lj && lj != 0xFFFFFFFFu) {
      const uint32_t c = atomicAdd(&C[j], 1u);
      if (c + 1u == (uint32_t)A.k) atomicMax(&A.thr[q], lj);
    }
  }
}

template <int CT, int D, int MODE>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs A) {
  constexpr int E = elem_bytes(CT);
  constexpr int NCH = chunks_per_block(CT, D);
  constexpr int RM = tile_frags(CT, D);
  constexpr int RG = RM >= 2 ? 2 : 1;  // fragments whose accumulators are live together
  constexpr int KSTEPS = (CT == MIPS_F32) ? D / 2 : (CT == MIPS_BF16 ? D / 16 : D / 64);
  constexpr int64_t BLK = block_bytes(CT, D);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // Workgroup -> (slice, query block). Dispatch places consecutive workgroups on
  // different XCDs; the query blocks of one slice share an XCD (and its L2).
  int slice, qblk;
  {
    const int w = blockIdx.x;
    if (A.nslices % 8 == 0) {
      const int xcd = w & 7, idx = w >> 3;
      slice = (idx / A.nqblk) * 8 + xcd;
      qblk = idx % A.nqblk;
    } else {
      slice = w / A.nqblk;
      qblk = w % A.nqblk;
    }
  }
  const int q0 = qblk * A.qb;
  const int nq = min(A.qb, A.b32 - q0);
  const int nqf = nq >> 5;

  // Stage the query block (already in operand layout) into LDS.
  {
    const u32x4_t* src = (const u32x4_t*)(A.qtile + (int64_t)q0 * D * E);
    u32x4_t* dst = (u32x4_t*)lds;
    const int n16 = nq * D * E / 16;
    for (int i = threadIdx.x; i < n16; i += kScoreThreads) dst[i] = src[i];
  }
  int* qexp_lds = (int*)(lds + (size_t)A.qb * D * E);
  float* thr_lds = (float*)(qexp_lds + A.qb) + wave * A.qb;
  if (CT == MIPS_FP8_E4M3)
    for (int i = threadIdx.x; i < nq; i += kScoreThreads) qexp_lds[i] = A.qexp[q0 + i];
  __syncthreads();

  const int64_t t_begin = (int64_t)slice * A.ntiles / A.nslices;
  const int64_t t_end = (int64_t)(slice + 1) * A.ntiles / A.nslices;

  for (int64_t t = t_begin + wave; t < t_end; t += kScoreWaves) {
    const int64_t f0 = t * RM;
    u32x4_t a[RM][NCH];
    int sa[RM];
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      const bool live = f0 + r < A.nfrag;
      const u32x4_t* p = (const u32x4_t*)(A.corpus + (f0 + r) * BLK) + lane;
#pragma unroll
      for (int c = 0; c < NCH; ++c) a[r][c] = live ? p[c * (kChunkBytes / 16)] : u32x4_t{0u, 0u, 0u, 0u};
      sa[r] = 127;
      if (CT == MIPS_FP8_E4M3 && live)
        sa[r] = (int)((__float_as_uint(A.row_scale[(f0 + r) * kFrag + (lane & 31)]) >> 23) & 0xFFu);
    }
    if (MODE == MODE_MAIN) {
      for (int i = lane; i < nq; i += kWave) {
        const int q = q0 + i;
        thr_lds[i] = q < A.b ? key_threshold(__hip_atomic_load(&A.thr[q], __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT))
                             : INFINITY;
      }
    }

    for (int qf = 0; qf < nqf; ++qf) {
      // The query fragment's whole B operand, loaded once from LDS.
      u32x4_t bq[NCH];
      const u32x4_t* bsrc = (const u32x4_t*)(lds + (size_t)qf * BLK) + lane;
#pragma unroll
      for (int c = 0; c < NCH; ++c) bq[c] = bsrc[c * (kChunkBytes / 16)];
      const int sb = (CT == MIPS_FP8_E4M3) ? qexp_lds[qf * 32 + (lane & 31)] : 127;
      const int ql = qf * 32 + (lane & 31);  // query within the block
      const int q = q0 + ql;
      const float T = (MODE == MODE_MAIN) ? thr_lds[ql] : 0.0f;

#pragma unroll
      for (int r0 = 0; r0 < RM; r0 += RG) {
        f32x16_t acc[RG];
#pragma unroll
        for (int g = 0; g < RG; ++g) acc[g] = f32x16_t{};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
          for (int g = 0; g < RG; ++g) mfma_step<CT>(acc[g], a[r0 + g], bq, sa[r0 + g], sb, s);

        if (MODE == MODE_SAMPLE) {
#pragma unroll
          for (int g = 0; g < RG; ++g) {
            const int64_t frag = f0 + r0 + g;
            const uint32_t word = (A.exclude && frag < A.nfrag) ? A.exclude[frag] : 0u;
            float m = neg_inf();
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int row = acc_row(i, lane);
              const bool ok = (frag * kFrag + row < A.n) && !((word >> row) & 1u);
              m = ok ? fmaxf(m, acc[g][i]) : m;
            }
            m = fmaxf(m, __shfl_xor(m, 32, kWave));
            if (lane < 32 && frag < A.G && q < A.b)
              A.delegates[(int64_t)q * A.G + frag] = (m == neg_inf()) ? 0u : score_key(m);
          }
        } else {
          float m = acc[0][0];
#pragma unroll
          for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int i = 0; i < 16; ++i) m = fmaxf(m, acc[g][i]);
          if (__ballot(m >= T)) {
            // Rare path: park this group's scores in a private array and a pass mask,
            // then append the set bits in one loop (keeps the unrolled code small so the
            // corpus operand stays in registers).
            float tv[RG * 16];
            uint32_t mask = 0u;
#pragma unroll
            for (int g = 0; g < RG; ++g)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                tv[g * 16 + i] = acc[g][i];
                mask |= (acc[g][i] >= T ? 1u : 0u) << (g * 16 + i);
              }
            if (q >= A.b) mask = 0u;
            while (mask) {
              const int bit = __builtin_ctz(mask);
              mask &= mask - 1u;
              const int64_t id = (f0 + r0 + (bit >> 4)) * kFrag + acc_row(bit & 15, lane);
              bool ok = id < A.n;
              if (ok && A.exclude) ok = !((A.exclude[id >> 5] >> (id & 31)) & 1u);
              if (ok) append_candidate(A, q, tv[bit], (uint32_t)id);
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ query prep
template <int CT, int QT, int D>
__global__ __launch_bounds__(64) void prep_queries_kernel(const void* __restrict__ queries, int b,
                                                          uint8_t* __restrict__ qtile,
                                                          int* __restrict__ qexp,
                                                          uint32_t* __restrict__ thr,
                                                          uint32_t* __restrict__ cnt,
                                                          uint32_t* __restrict__ lvl,
                                                          uint32_t* __restrict__ lcnt) {
  constexpr int NCH = chunks_per_block(CT, D);
  const int lane = threadIdx.x;
  const int q = blockIdx.x * kFrag + (lane & 31);
  const bool live = q < b;
  auto val = [&](int dim) -> float {
    if (!live) return 0.0f;
    if (QT == MIPS_F32) return ((const float*)queries)[(int64_t)q * D + dim];
    return bf16_to_f32(((const uint16_t*)queries)[(int64_t)q * D + dim]);
  };
  float sinv = 1.0f;
  if (CT == MIPS_FP8_E4M3) {
    float m = 0.0f;
    for (int j = 0; j < D; ++j) m = fmaxf(m, fabsf(val(j)));
    int t = e4m3_scale_exp(m);
    t = t < -126 ? -126 : (t > 127 ? 127 : t);
    sinv = exp2_int(-t);
    if (lane < 32) qexp[q] = t + 127;
  }
  uint8_t* out = qtile + (int64_t)blockIdx.x * block_bytes(CT, D);
  for (int c = 0; c < NCH; ++c) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (CT == MIPS_F32) {
      for (int t = 0; t < 4; ++t) v[t] = __float_as_uint(val(slot_dim(CT, c, lane, t)));
    } else if (CT == MIPS_BF16) {
      for (int t = 0; t < 8; t += 2)
        v[t >> 1] = (uint32_t)f32_to_bf16(val(slot_dim(CT, c, lane, t))) |
                    ((uint32_t)f32_to_bf16(val(slot_dim(CT, c, lane, t + 1))) << 16);
    } else {
      for (int t = 0; t < 16; ++t)
        v[t >> 2] |= (uint32_t)f32_to_e4m3(val(slot_dim(CT, c, lane, t)) * sinv) << (8 * (t & 3));
    }
    *(u32x4_t*)(out + (int64_t)c * kChunkBytes + lane * 16) = v;
  }
  if (lane < 32 && live) {
    thr[q] = 0u;
    cnt[q] = 0u;
    for (int j = 0; j < kLevels; ++j) {
      lvl[(int64_t)q * kLevels + j] = 0xFFFFFFFFu;
      lcnt[(int64_t)q * kLevels + j] = 0u;
    }
  }
}

// --------------------------------------------------------------- radix select
// r-th largest (r >= 1) of n 32-bit keys in LDS, by four 8-bit digit passes.
__device__ uint32_t select_rth_u32(const uint32_t* keys, int n, int r, uint32_t* hist,
                                   uint32_t* shared2) {
  uint32_t prefix = 0u, mask = 0u;
  int rem = r;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t acc = 0u, dsel = 0u;
      for (int dg = 255; dg >= 0; --dg) {
        if (acc + hist[dg] >= (uint32_t)rem) {
          dsel = (uint32_t)dg;
          break;
        }
        acc += hist[dg];
      }
      shared2[0] = dsel;
      shared2[1] = (uint32_t)rem - acc;
    }
    __syncthreads();
    prefix |= shared2[0] << shift;
    mask |= 255u << shift;
    rem = (int)shared2[1];
    __syncthreads();
  }
  return prefix;
}

// Descending bitonic sort of p (power of two) 64-bit keys in LDS.
__device__ void bitonic_desc(uint64_t* s, int p) {
  for (int size = 2; size <= p; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (p >> 1); i += blockDim.x) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = s[lo], y = s[hi];
        if ((x < y) == desc) {
          s[lo] = y;
          s[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Per query: the K-th largest delegate becomes the starting threshold; the delegates
// of rank K/2, K/4, ... become the levels.
__global__ __launch_bounds__(kSelThreads) void sample_threshold_kernel(const uint32_t* __restrict__ del,
                                                                       int G, int b, int k,
                                                                       uint32_t* __restrict__ thr,
                                                                       uint32_t* __restrict__ lvl) {
  __shared__ uint32_t keys[kSampleGroups];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  __shared__ uint64_t top[2048];
  __shared__ uint32_t ntop;
  const int q = blockIdx.x;
  if (q >= b) return;
  for (int i = threadIdx.x; i < G; i += blockDim.x) keys[i] = del[(int64_t)q * G + i];
  if (threadIdx.x == 0) ntop = 0u;
  __syncthreads();
  uint32_t kth = 0u;
  if (G >= k) kth = select_rth_u32(keys, G, k, hist, sh);
  // Gather the delegates >= kth (ties may give more than k; keep at most 2048).
  for (int i = threadIdx.x; i < G; i += blockDim.x) {
    if (keys[i] >= kth && keys[i] != 0u) {
      const uint32_t slot = atomicAdd(&ntop, 1u);
      if (slot < 2048u) top[slot] = keys[i];
    }
  }
  __syncthreads();
  const int m = (int)min(ntop, 2048u);
  for (int i = m + threadIdx.x; i < 2048; i += blockDim.x) top[i] = 0u;
  __syncthreads();
  bitonic_desc(top, 2048);
  if (threadIdx.x == 0) {
    thr[q] = kth;
    for (int j = 0; j < kLevels; ++j) {
      const int rank = k >> (j + 1);
      uint32_t v = 0xFFFFFFFFu;
      if (rank >= 1 && rank <= m) v = (uint32_t)top[rank - 1];
      if (v == 0u) v = 0xFFFFFFFFu;
      lvl[(int64_t)q * kLevels + j] = v;
    }
  }
}

// ---------------------------------------------------------------- final select
struct SelectArgs {
  const uint8_t* corpus;
  const float* row_scale;
  const uint32_t* exclude;
  const uint8_t* qtile;
  const int* qexp;
  int64_t n;
  int b;
  int k;
  int64_t cap;
  const uint32_t* cnt;
  const uint64_t* cand;
  float* out_scores;
  int32_t* out_ids;
};

// Selection state of select_top: keys with (key & mask) >= prefix are the r best.
struct Sel64 {
  uint64_t prefix, mask;
};

// The r best of n unique 64-bit keys (1 <= r <= n), MSD radix with 8-bit digits; stops
// as soon as the boundary digit's bin holds exactly the remaining count.
template <typename Get>
__device__ Sel64 select_top(Get get, int64_t n, int r, uint32_t* hist, uint64_t* sh) {
  uint64_t prefix = 0u, mask = 0u;
  int64_t rem = r;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
      const uint64_t key = get(i);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t acc = 0;
      int dsel = 0;
      for (int dg = 255; dg >= 0; --dg) {
        if (acc + (int64_t)hist[dg] >= rem) {
          dsel = dg;
          break;
        }
        acc += hist[dg];
      }
      sh[0] = (uint64_t)dsel;
      sh[1] = (uint64_t)(rem - acc);
      sh[2] = hist[dsel];
    }
    __syncthreads();
    prefix |= sh[0] << shift;
    mask |= 255ull << shift;
    rem = (int64_t)sh[1];
    const bool done = sh[2] == sh[1];
    __syncthreads();
    if (done) break;
  }
  return Sel64{prefix, mask};
}

// Writes the (already gathered, sorted descending) keys of query q, padding the rest.
__device__ void write_out(const SelectArgs& A, int q, const uint64_t* s, int cnt) {
  for (int t = threadIdx.x; t < A.k; t += blockDim.x) {
    float sc = -INFINITY;
    int32_t id = -1;
    if (t < cnt) {
      sc = key_score((uint32_t)(s[t] >> 32));
      id = (int32_t)composite_id(s[t]);
    }
    A.out_scores[(int64_t)q * A.k + t] = sc;
    A.out_ids[(int64_t)q * A.k + t] = id;
  }
}

__device__ __forceinline__ int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Exact rescan of query q when its candidate list overflowed: VALU dot products in
// dimension order, a candidate buffer in LDS pruned by a composite threshold.
template <int CT, int D>
__device__ void fallback_scan(const SelectArgs& A, int q, uint64_t start_thr, uint64_t* buf,
                              uint32_t* hist, uint64_t* sh, float* qv) {
  __shared__ uint32_t nbuf;
  const int lane_t = threadIdx.x;
  // Query values in fp32 (fp8: code * 2^t, exact).
  for (int j = lane_t; j < D; j += blockDim.x) {
    const int64_t off = (int64_t)(q >> 5) * block_bytes(CT, D) +
                        (packed_offset(CT, D, q & 31, j));
    float v;
    if (CT == MIPS_F32)
      v = *(const float*)(A.qtile + off);
    else if (CT == MIPS_BF16)
      v = bf16_to_f32(*(const uint16_t*)(A.qtile + off));
    else
      v = e4m3_to_f32(A.qtile[off]) * exp2_int(A.qexp[q] - 127);
    qv[j] = v;
  }
  if (threadIdx.x == 0) nbuf = 0u;
  __syncthreads();
  uint64_t thr = start_thr;
  const int round = blockDim.x * 4;
  for (int64_t base = 0; base < A.n; base += round) {
    if (nbuf + (uint32_t)round > (uint32_t)kFallbackBuf) {
      const int m = (int)nbuf;
      const int r = min(A.k, m);
      const Sel64 sel = select_top([&](int64_t i) { return buf[i]; }, m, r, hist, sh);
      __syncthreads();
      if (threadIdx.x == 0) nbuf = 0u;
      __syncthreads();
      // Compact in place through a second pass: keep the r selected keys.
      uint64_t mine[kFallbackBuf / kSelThreads];
      int nm = 0;
      for (int i = threadIdx.x; i < m; i += blockDim.x) mine[nm++] = buf[i];
      __syncthreads();
      for (int t = 0; t < nm; ++t)
        if ((mine[t] & sel.mask) >= sel.prefix) buf[atomicAdd(&nbuf, 1u)] = mine[t];
      __syncthreads();
      // New threshold: the smallest kept key once k are held.
      if ((int)nbuf >= A.k) {
        uint64_t lo = ~0ull;
        for (int i = 0; i < (int)nbuf; ++i) lo = buf[i] < lo ? buf[i] : lo;
        thr = lo > thr ? lo : thr;
      }
      __syncthreads();
    }
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + (int64_t)u * blockDim.x + threadIdx.x;
      if (i >= A.n) continue;
      if (A.exclude && ((A.exclude[i >> 5] >> (i & 31)) & 1u)) continue;
      float s = 0.0f;
      float rs = 1.0f;
      if (CT == MIPS_FP8_E4M3) rs = A.row_scale[i];
      for (int j = 0; j < D; ++j) {
        const int64_t off = packed_offset(CT, D, i, j);
        float c;
        if (CT == MIPS_F32)
          c = *(const float*)(A.corpus + off);
        else if (CT == MIPS_BF16)
          c = bf16_to_f32(*(const uint16_t*)(A.corpus + off));
        else
          c = e4m3_to_f32(A.corpus[off]);
        s = fmaf(qv[j], c, s);
      }
      if (CT == MIPS_FP8_E4M3) s *= rs;
      const uint64_t key = composite(score_key(s), (uint32_t)i);
      if (key >= thr) buf[atomicAdd(&nbuf, 1u)] = key;
    }
    __syncthreads();
  }
  const int m = (int)nbuf;
  const int r = min(A.k, m);
  __shared__ uint32_t nsel;
  if (threadIdx.x == 0) nsel = 0u;
  __syncthreads();
  if (r > 0) {
    const Sel64 sel = select_top([&](int64_t i) { return buf[i]; }, m, r, hist, sh);
    uint64_t mine[kFallbackBuf / kSelThreads];
    int nm = 0;
    for (int i = threadIdx.x; i < m; i += blockDim.x) mine[nm++] = buf[i];
    __syncthreads();
    for (int t = 0; t < nm; ++t)
      if ((mine[t] & sel.mask) >= sel.prefix) buf[atomicAdd(&nsel, 1u)] = mine[t];
    __syncthreads();
  }
  const int p = pow2_at_least(r < 2 ? 2 : r);
  for (int i = r + threadIdx.x; i < p; i += blockDim.x) buf[i] = 0u;
  __syncthreads();
  bitonic_desc(buf, p);
  write_out(A, q, buf, r);
}

template <int CT, int D>
__global__ __launch_bounds__(kSelThreads) void final_select_kernel(SelectArgs A) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t sh[4];
  __shared__ uint64_t buf[kFallbackBuf];
  __shared__ float qv[D];
  __shared__ uint32_t ngot;
  const int q = blockIdx.x;
  if (q >= A.b) return;
  const int64_t c = A.cnt[q];
  const uint64_t* list = A.cand + (int64_t)q * A.cap;
  if (c > A.cap) {
    // Overflow: the stored entries are still valid candidates, so their k-th best is
    // a lower bound for the exact rescan.
    uint64_t start = 0u;
    if (A.cap >= A.k) {
      const Sel64 sel = select_top([&](int64_t i) { return list[i]; }, A.cap, A.k, hist, sh);
      // The k-th best stored key is the smallest key with (key & mask) >= prefix;
      // prefix itself is a lower bound of it.
      start = sel.prefix;
    }
    __syncthreads();
    fallback_scan<CT, D>(A, q, start, buf, hist, sh, qv);
    return;
  }
  const int r = (int)min<int64_t>(c, A.k);
  if (threadIdx.x == 0) ngot = 0u;
  __syncthreads();
  if (r > 0) {
    Sel64 sel{0u, 0u};
    if (c > r) sel = select_top([&](int64_t i) { return list[i]; }, c, r, hist, sh);
    for (int64_t i = threadIdx.x; i < c; i += blockDim.x) {
      const uint64_t key = list[i];
      if ((key & sel.mask) >= sel.prefix) buf[atomicAdd(&ngot, 1u)] = key;
    }
    __syncthreads();
  }
  const int p = pow2_at_least(r < 2 ? 2 : r);
  for (int i = r + threadIdx.x; i < p; i += blockDim.x) buf[i] = 0u;
  __syncthreads();
  bitonic_desc(buf, p);
  write_out(A, q, buf, r);
}

// ------------------------------------------------------------------- planning
struct Plan {
  int b, b32, k, d, qdt, cdt;
  int64_t n, n32;
  int rm, qb, nqblk, G;
  int64_t ntiles, cap;
  size_t off_qtile, off_qexp, off_thr, off_cnt, off_lvl, off_lcnt, off_del, off_cand, fixed;
  size_t lds_score;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int64_t default_cap(int64_t n32, int k) {
  const int64_t want = std::max<int64_t>(16 * (int64_t)k, 32768);
  return std::min<int64_t>(n32 * kFrag, want);
}

static void make_plan(Plan& p, int b, int64_t n, int d, int k, int qdt, int cdt) {
  p.b = b;
  p.b32 = (b + 31) / 32 * 32;
  p.k = k;
  p.d = d;
  p.qdt = qdt;
  p.cdt = cdt;
  p.n = n;
  p.n32 = (n + 31) / 32;
  p.rm = tile_frags(cdt, d);
  p.ntiles = (p.n32 + p.rm - 1) / p.rm;
  const int E = elem_bytes(cdt);
  // LDS per query: its operand row, its fp8 exponent and one threshold per wave.
  int qb = kLdsScoreBudget / (d * E + 4 + 4 * kScoreWaves);
  qb = qb / 32 * 32;
  if (qb > 2048) qb = 2048;
  if (qb > p.b32) qb = p.b32;
  p.nqblk = (p.b32 + qb - 1) / qb;
  p.qb = ((p.b32 + p.nqblk - 1) / p.nqblk + 31) / 32 * 32;
  p.lds_score = (size_t)p.qb * d * E + (size_t)p.qb * 4 + (size_t)kScoreWaves * p.qb * 4;
  size_t o = 0;
  p.off_qtile = o;
  o = align256(o + (size_t)p.b32 * d * E);
  p.off_qexp = o;
  o = align256(o + (size_t)p.b32 * 4);
  p.off_thr = o;
  o = align256(o + (size_t)b * 4);
  p.off_cnt = o;
  o = align256(o + (size_t)b * 4);
  p.off_lvl = o;
  o = align256(o + (size_t)b * kLevels * 4);
  p.off_lcnt = o;
  o = align256(o + (size_t)b * kLevels * 4);
  p.off_del = o;
  p.G = (int)std::min<int64_t>(p.n32, kSampleGroups);
  o = align256(o + (size_t)b * p.G * 4);
  p.off_cand = o;
  p.fixed = o;
}

template <int CT, int D>
static int run_topk(const Plan& p, const void* queries, const void* corpus, const float* row_scale,
                    const uint32_t* exclude, float* out_scores, int32_t* out_ids, uint8_t* ws,
                    hipStream_t s) {
  uint8_t* qtile = ws + p.off_qtile;
  int* qexp = (int*)(ws + p.off_qexp);
  uint32_t* thr = (uint32_t*)(ws + p.off_thr);
  uint32_t* cnt = (uint32_t*)(ws + p.off_cnt);
  uint32_t* lvl = (uint32_t*)(ws + p.off_lvl);
  uint32_t* lcnt = (uint32_t*)(ws + p.off_lcnt);
  uint32_t* del = (uint32_t*)(ws + p.off_del);
  uint64_t* cand = (uint64_t*)(ws + p.off_cand);

  if (p.qdt == MIPS_F32)
    hipLaunchKernelGGL((prep_queries_kernel<CT, MIPS_F32, D>), dim3(p.b32 / 32), dim3(64), 0, s,
                       queries, p.b, qtile, qexp, thr, cnt, lvl, lcnt);
  else
    hipLaunchKernelGGL((prep_queries_kernel<CT, MIPS_BF16, D>), dim3(p.b32 / 32), dim3(64), 0, s,
                       queries, p.b, qtile, qexp, thr, cnt, lvl, lcnt);
  int rc = check_launch();
  if (rc) return rc;

  static bool lds_set[2] = {false, false};
  if (!lds_set[0]) {
    (void)hipFuncSetAttribute((const void*)score_kernel<CT, D, MODE_SAMPLE>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)hipFuncSetAttribute((const void*)score_kernel<CT, D, MODE_MAIN>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    lds_set[0] = true;
  }
  (void)lds_set[1];

  ScoreArgs A;
  A.corpus = (const uint8_t*)corpus;
  A.row_scale = row_scale;
  A.exclude = exclude;
  A.qtile = qtile;
  A.qexp = qexp;
  A.n = p.n;
  A.n32 = p.n32;
  A.b = p.b;
  A.b32 = p.b32;
  A.qb = p.qb;
  A.nqblk = p.nqblk;
  A.k = p.k;
  A.cap = p.cap;
  A.thr = thr;
  A.lvl = lvl;
  A.lcnt = lcnt;
  A.cnt = cnt;
  A.cand = cand;
  A.delegates = del;
  A.G = p.G;

  const int cus = device_cu_count();
  auto slices_for = [&](int64_t ntiles) {
    int64_t want = std::max<int64_t>(1, cus / p.nqblk);
    if (want >= 8) want = want / 8 * 8;
    return (int)std::max<int64_t>(1, std::min<int64_t>(ntiles, want));
  };

  // Without a sampled threshold every item is a candidate, which is only allowed when the
  // lists cannot overflow, and only worth it for small corpora.
  const bool sample = p.n32 * kFrag > p.cap || p.n32 * kFrag > 8 * (int64_t)p.k + 4096;
  if (sample) {
    A.nfrag = p.G;
    A.ntiles = (p.G + p.rm - 1) / p.rm;
    A.nslices = slices_for(A.ntiles);
    hipLaunchKernelGGL((score_kernel<CT, D, MODE_SAMPLE>), dim3(A.nslices * p.nqblk),
                       dim3(kScoreThreads), p.lds_score, s, A);
    if ((rc = check_launch())) return rc;
    hipLaunchKernelGGL(sample_threshold_kernel, dim3(p.b), dim3(kSelThreads), 0, s, del, p.G, p.b,
                       p.k, thr, lvl);
    if ((rc = check_launch())) return rc;
  }

  A.nfrag = p.n32;
  A.ntiles = p.ntiles;
  A.nslices = slices_for(A.ntiles);
  hipEvent_t ev0, ev1;
  timing_events(&ev0, &ev1);
  if (ev0) (void)hipEventRecord(ev0, s);
  hipLaunchKernelGGL((score_kernel<CT, D, MODE_MAIN>), dim3(A.nslices * p.nqblk),
                     dim3(kScoreThreads), p.lds_score, s, A);
  if ((rc = check_launch())) return rc;
  if (ev1) (void)hipEventRecord(ev1, s);

  SelectArgs S;
  S.corpus = (const uint8_t*)corpus;
  S.row_scale = row_scale;
  S.exclude = exclude;
  S.qtile = qtile;
  S.qexp = qexp;
  S.n = p.n;
  S.b = p.b;
  S.k = p.k;
  S.cap = p.cap;
  S.cnt = cnt;
  S.cand = cand;
  S.out_scores = out_scores;
  S.out_ids = out_ids;
  hipLaunchKernelGGL((final_select_kernel<CT, D>), dim3(p.b), dim3(kSelThreads), 0, s, S);
  return check_launch();
}

template <int CT>
static int dispatch_d(const Plan& p, const void* queries, const void* corpus,
                      const float* row_scale, const uint32_t* exclude, float* out_scores,
                      int32_t* out_ids, uint8_t* ws, hipStream_t s) {
#define MIPS_RUN(DD) return run_topk<CT, DD>(p, queries, corpus, row_scale, exclude, out_scores, out_ids, ws, s)
  switch (p.d) {
    case 16: if constexpr (CT != MIPS_FP8_E4M3) { MIPS_RUN(16); } break;
    case 32: if constexpr (CT != MIPS_FP8_E4M3) { MIPS_RUN(32); } break;
    case 64: MIPS_RUN(64);
    case 128: MIPS_RUN(128);
    case 256: MIPS_RUN(256);
  }
#undef MIPS_RUN
  return MIPS_ERR_UNSUPPORTED;
}

static int validate_topk(const void* queries, int32_t qdt, int32_t b, const void* corpus,
                         const float* row_scale, int32_t cdt, int64_t n, int32_t d,
                         int32_t k) {
  if (qdt != MIPS_F32 && qdt != MIPS_BF16) return MIPS_ERR_UNSUPPORTED;
  if (cdt != MIPS_F32 && cdt != MIPS_BF16 && cdt != MIPS_FP8_E4M3) return MIPS_ERR_UNSUPPORTED;
  if (cdt == MIPS_F32 && qdt != MIPS_F32) return MIPS_ERR_UNSUPPORTED;
  if (b < 1 || n < 1 || n > (int64_t)0x7FFFFFFF - 64 || k < 1) return MIPS_ERR_INVALID_ARG;
  if (k > MIPS_K_MAX) return MIPS_ERR_UNSUPPORTED;
  if (!corpus_d_supported(cdt, d)) return MIPS_ERR_UNSUPPORTED;
  (void)queries;
  (void)corpus;
  (void)row_scale;
  return MIPS_OK;
}

}  // namespace mips

extern "C" {

size_t mips_topk_workspace_size(int32_t b, int64_t n, int32_t d, int32_t k, int32_t query_dtype,
                                int32_t corpus_dtype) {
  if (mips::validate_topk(nullptr, query_dtype, b, nullptr, nullptr, corpus_dtype, n, d, k) !=
      MIPS_OK)
    return 0;
  mips::Plan p;
  mips::make_plan(p, b, n, d, k, query_dtype, corpus_dtype);
  const int64_t cap = mips::default_cap(p.n32, k);
  return p.fixed + (size_t)b * (size_t)cap * 8u;
}

int mips_topk(const void* queries, int32_t query_dtype, int32_t b, const void* corpus,
              const float* row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
              const uint32_t* exclude, int32_t k, float* out_scores, int32_t* out_ids,
              void* workspace, size_t workspace_bytes, void* stream) {
  if (!queries || !corpus || !out_scores || !out_ids || !workspace) return MIPS_ERR_INVALID_ARG;
  const int rc0 =
      mips::validate_topk(queries, query_dtype, b, corpus, row_scale, corpus_dtype, n, d, k);
  if (rc0 != MIPS_OK) return rc0;
  if (corpus_dtype == MIPS_FP8_E4M3 && !row_scale) return MIPS_ERR_INVALID_ARG;
  if (!mips::aligned(queries, 4) || !mips::aligned(corpus, 16) || !mips::aligned(workspace, 256) ||
      !mips::aligned(out_scores, 4) || !mips::aligned(out_ids, 4) ||
      (exclude && !mips::aligned(exclude, 4)) || (row_scale && !mips::aligned(row_scale, 4)))
    return MIPS_ERR_INVALID_ARG;
  mips::Plan p;
  mips::make_plan(p, b, n, d, k, query_dtype, corpus_dtype);
  if (workspace_bytes < p.fixed) return MIPS_ERR_WORKSPACE;
  int64_t cap = (int64_t)((workspace_bytes - p.fixed) / ((size_t)b * 8u));
  cap = std::min<int64_t>(cap, p.n32 * 32);
  if (cap < std::min<int64_t>(n, k)) return MIPS_ERR_WORKSPACE;
  p.cap = cap;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  switch (corpus_dtype) {
    case MIPS_F32:
      return mips::dispatch_d<MIPS_F32>(p, queries, corpus, row_scale, exclude, out_scores, out_ids, ws, s);
    case MIPS_BF16:
      return mips::dispatch_d<MIPS_BF16>(p, queries, corpus, row_scale, exclude, out_scores, out_ids, ws, s);
    default:
      return mips::dispatch_d<MIPS_FP8_E4M3>(p, queries, corpus, row_scale, exclude, out_scores, out_ids, ws, s);
  }
}

}  // extern "C"
