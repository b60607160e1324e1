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

constexpr int kLevels = 12;         // threshold levels per query
constexpr int kScoreThreads = 256;  // 4 waves: one per SIMD, up to 512 registers each
constexpr int kScoreWaves = kScoreThreads / kWave;
constexpr int kSampleGroups = 8192; // delegates per query (prefix sample of 8192 blocks)
constexpr int kSelThreads = 256;
constexpr int kLdsScoreBudget = 150 * 1024;  // query block + scales + thresholds + staging
constexpr int kStageCap = 384;               // staged survivors per wave
constexpr int kStageBurst = 256;             // room kept free before each group
constexpr int kMaxQueryBlock = 512;          // queries staged in LDS per workgroup
constexpr int kRefreshRegs = kMaxQueryBlock / kScoreThreads;  // threshold loads per lane

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
  uint32_t* ovf;
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

// Appends one survivor (composite key) of query q and counts it against the query's
// levels L (ascending where set): once K survivors at or above level j exist, level j
// is a valid threshold and is published with atomicMax.
__device__ __forceinline__ void append_candidate(const ScoreArgs& A, int q, uint64_t ckey,
                                                 const uint32_t* L) {
  const uint32_t key = (uint32_t)(ckey >> 32);
  const uint32_t pos = atomicAdd(&A.cnt[q], 1u);
  if ((int64_t)pos < A.cap) A.cand[(int64_t)q * A.cap + pos] = ckey;
  uint32_t* C = A.lcnt + (int64_t)q * kLevels;
  uint32_t res[kLevels];
#pragma unroll
  for (int j = 0; j < kLevels; ++j)
    if (key >= L[j] && L[j] != 0xFFFFFFFFu) res[j] = atomicAdd(&C[j], 1u);
#pragma unroll
  for (int j = 0; j < kLevels; ++j)
    if (key >= L[j] && L[j] != 0xFFFFFFFFu && res[j] + 1u == (uint32_t)A.k)
      atomicMax(&A.thr[q], L[j]);
}

__device__ __forceinline__ bool is_excluded(const uint32_t* bits, int64_t id) {
  return bits && ((bits[id >> 5] >> (id & 31)) & 1u);
}

// Appends a wave's staged survivors (one entry per lane per round).
__device__ __forceinline__ void flush_staged(const uint64_t* st_key, const uint16_t* st_q, int nst,
                                          int q0, const uint32_t* lvl_lds, int64_t n,
                                          const uint32_t* exclude, uint32_t* cnt, uint64_t* cand,
                                          int64_t cap, uint32_t* lcnt, uint32_t* thr, int k) {
  const int lane = threadIdx.x & 63;
  for (int e = lane; e < nst; e += kWave) {
    const uint64_t ck = st_key[e];
    const int64_t id = composite_id(ck);
    const int ql = st_q[e];
    if (id >= n || is_excluded(exclude, id)) continue;
    const int q = q0 + ql;
    const uint32_t* L = lvl_lds + ql * kLevels;
    const uint32_t key = (uint32_t)(ck >> 32);
    const uint32_t pos = atomicAdd(&cnt[q], 1u);
    if ((int64_t)pos < cap) cand[(int64_t)q * cap + pos] = ck;
    uint32_t* C = lcnt + (int64_t)q * kLevels;
    for (int j = 0; j < kLevels; ++j) {
      const uint32_t lj = L[j];
      if (lj == 0xFFFFFFFFu || key < lj) continue;
      if (atomicAdd(&C[j], 1u) + 1u == (uint32_t)k) atomicMax(&thr[q], lj);
    }
  }
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// Corpus fragments per pipeline stage: at most 2 (16 KiB of corpus per wave and stage for
// 256-byte rows), so that two stages of corpus operand, two query operands and two sets of
// accumulators fit one wave's 512 registers.
__host__ __device__ constexpr int stage_frags(int ct, int d) {
  const int r = 512 / (d * elem_bytes(ct));
  return r < 1 ? 1 : (r > 2 ? 2 : r);
}

template <int CT, int D, int MODE>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs A) {
  constexpr int E = elem_bytes(CT);
  constexpr int NCH = chunks_per_block(CT, D);
  constexpr int RM = stage_frags(CT, D);
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

  // LDS: query block operand | fp8 query exponents | thresholds (shared by the waves) |
  // levels | per-wave survivor staging (composite keys, query index).
  {
    const u32x4_t* src = (const u32x4_t*)(A.qtile + (int64_t)q0 * D * E);
    u32x4_t* dst = (u32x4_t*)lds;
    const int n16 = nq * D * E / 16;
    for (int i = threadIdx.x; i < n16; i += kScoreThreads) dst[i] = src[i];
  }
  int* qexp_lds = (int*)(lds + (size_t)A.qb * D * E);
  float* thr_lds = (float*)(qexp_lds + A.qb);
  uint32_t* lvl_lds = (uint32_t*)(thr_lds + A.qb);
  uint64_t* st_key = (uint64_t*)(lvl_lds + (size_t)A.qb * kLevels) + wave * kStageCap;
  uint16_t* st_q = (uint16_t*)((uint64_t*)(lvl_lds + (size_t)A.qb * kLevels) +
                               kScoreWaves * kStageCap) + wave * kStageCap;
  if (CT == MIPS_FP8_E4M3)
    for (int i = threadIdx.x; i < nq; i += kScoreThreads) qexp_lds[i] = A.qexp[q0 + i];
  if (MODE == MODE_MAIN) {
    for (int i = threadIdx.x; i < nq; i += kScoreThreads) {
      const int q = q0 + i;
      thr_lds[i] = q < A.b ? key_threshold(A.thr[q]) : INFINITY;
    }
    for (int i = threadIdx.x; i < nq * kLevels; i += kScoreThreads) {
      const int q = q0 + i / kLevels;
      lvl_lds[i] = q < A.b ? A.lvl[(int64_t)q * kLevels + (i % kLevels)] : 0xFFFFFFFFu;
    }
  }
  __syncthreads();

  int st_n = 0;  // staged survivors of this wave (wave-uniform; may exceed the capacity)
  auto flush = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    flush_staged(st_key, st_q, min(st_n, kStageCap), q0, lvl_lds, A.n, A.exclude, A.cnt, A.cand,
                 A.cap, A.lcnt, A.thr, A.k);
    __builtin_amdgcn_wave_barrier();
    st_n = 0;
  };

  // Threshold refresh: each wave refreshes its slice of the shared LDS copy. Any published
  // threshold is valid, so the other waves may read a copy that is one refresh old.
  uint32_t rv[kRefreshRegs];
  auto refresh_issue = [&]() {
#pragma unroll
    for (int r = 0; r < kRefreshRegs; ++r) {
      const int i = min(threadIdx.x + r * kScoreThreads, nq - 1);
      rv[r] = __hip_atomic_load(&A.thr[min(q0 + i, A.b - 1)], __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto refresh_commit = [&]() {
#pragma unroll
    for (int r = 0; r < kRefreshRegs; ++r) {
      const int i = threadIdx.x + r * kScoreThreads;
      if (i < nq && q0 + i < A.b) thr_lds[i] = key_threshold(rv[r]);
    }
  };

  // A stage's loads are unconditional: fragments past the end read the last block again
  // (their ids are >= n and never survive), so the compiler's wait counts stay exact.
  auto load_stage = [&](u32x4_t (&a)[RM][NCH], int (&sa)[RM], uint32_t (&wd)[RM], int64_t f0) {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      const int64_t fr = min<int64_t>(f0 + r, A.n32 - 1);
      const u32x4_t* p = (const u32x4_t*)(A.corpus + fr * BLK) + lane;
#pragma unroll
      for (int c = 0; c < NCH; ++c) a[r][c] = p[c * (kChunkBytes / 16)];
      sa[r] = 127;
      if (CT == MIPS_FP8_E4M3)
        sa[r] = (int)((__float_as_uint(A.row_scale[fr * kFrag + (lane & 31)]) >> 23) & 0xFFu);
      wd[r] = 0u;
      if (MODE == MODE_SAMPLE && A.exclude) wd[r] = A.exclude[fr];
    }
  };

  // A query fragment's B operand and this lane's threshold, read from LDS one fragment
  // ahead of their use.
  auto load_b = [&](u32x4_t (&bq)[NCH], float& T, int qf) {
    const u32x4_t* bsrc = (const u32x4_t*)(lds + (size_t)qf * BLK) + lane;
#pragma unroll
    for (int c = 0; c < NCH; ++c) bq[c] = bsrc[c * (kChunkBytes / 16)];
    T = (MODE == MODE_MAIN) ? thr_lds[qf * 32 + (lane & 31)] : 0.0f;
  };
  auto mfmas = [&](f32x16_t (&acc)[RM], const u32x4_t (&a)[RM][NCH], const int (&sa)[RM],
                   const u32x4_t (&bq)[NCH], int qf) {
    const int sb = (CT == MIPS_FP8_E4M3) ? qexp_lds[qf * 32 + (lane & 31)] : 127;
#pragma unroll
    for (int g = 0; g < RM; ++g) acc[g] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int g = 0; g < RM; ++g) mfma_step<CT>(acc[g], a[g], bq, sa[g], sb, s);
  };

  // Epilogue of one query fragment against the stage's RM corpus fragments.
  // Sample mode: per-(query, block) maxima. Main mode, fast part: one max per fragment
  // (16 scores per lane) and a ballot of `max >= threshold`, branch-free so it can be
  // interleaved with the next fragment's MFMAs.
  auto epi_sample = [&](const f32x16_t (&acc)[RM], const uint32_t (&wd)[RM], int64_t f0, int qf) {
    const int q = q0 + qf * 32 + (lane & 31);
#pragma unroll
    for (int g = 0; g < RM; ++g) {
      const int64_t frag = f0 + g;
      const uint32_t word = wd[g];
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
  };
  auto epi_fast = [&](const f32x16_t (&acc)[RM], const float T, uint64_t (&hit)[RM]) {
#pragma unroll
    for (int g = 0; g < RM; ++g) {
      float m = acc[g][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) m = fmaxf(m, acc[g][i]);
      hit[g] = __ballot(m >= T);
    }
  };
  // Rare part: a fragment that cleared the threshold is resolved by 4-row blocks, then
  // value by value with ballot + mbcnt compaction into the wave's staging buffer. The
  // block and value loops index the accumulators with a wave-uniform runtime index and
  // stay rolled, so the rare path adds little code to the MFMA loop.
  auto epi_slow = [&](const f32x16_t (&acc)[RM], const uint64_t (&hit)[RM], int64_t f0, int qf,
                      const float T) {
    const int ql = qf * 32 + (lane & 31);  // query within the block
    const int q = q0 + ql;
#pragma unroll
    for (int g = 0; g < RM; ++g) {
      if (!hit[g]) continue;
      const int64_t frag = f0 + g;
#pragma unroll 1
      for (int bb = 0; bb < 4; ++bb) {
        const float pm = fmaxf(fmaxf(acc[g][4 * bb], acc[g][4 * bb + 1]),
                               fmaxf(acc[g][4 * bb + 2], acc[g][4 * bb + 3]));
        if (!__ballot(pm >= T)) continue;
#pragma unroll 1
        for (int i = 4 * bb; i < 4 * bb + 4; ++i) {
          const float v = acc[g][i];
          const bool pass = v >= T && q < A.b;
          const uint64_t bm = __ballot(pass);
          if (!bm) continue;
          const int pos = st_n + (int)__builtin_amdgcn_mbcnt_hi(
                                     (uint32_t)(bm >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
          if (pass) {
            const int64_t id = frag * kFrag + acc_row(i, lane);
            if (pos < kStageCap) {
              st_key[pos] = composite(score_key(v), (uint32_t)id);
              st_q[pos] = (uint16_t)ql;
            } else {
              atomicOr(&A.ovf[q], 1u);  // no room: the query is rescanned exactly
            }
          }
          st_n += __popcll(bm);
        }
      }
    }
  };

  // One stage against every query fragment, software-pipelined over the fragments: the
  // MFMAs of fragment qf+1 and the LDS reads of fragment qf+2's operand are issued before
  // the epilogue of fragment qf, so the epilogue (and its rare path) runs while the matrix
  // pipe works on the next fragment.
  auto compute_stage = [&](const u32x4_t (&a)[RM][NCH], const int (&sa)[RM],
                           const uint32_t (&wd)[RM], int64_t f0) {
    u32x4_t b0[NCH], b1[NCH];
    f32x16_t c0[RM], c1[RM];
    uint64_t hit[RM];
    float t0, t1, tc0, tc1;  // thresholds: loaded (t*) and in use (tc*)
    load_b(b0, t0, 0);
    load_b(b1, t1, min(1, nqf - 1));
    mfmas(c0, a, sa, b0, 0);
    tc0 = t0;
    int qf = 0;
    for (;;) {
      // c0 holds fragment qf; b1 holds fragment qf+1's operand.
      if (MODE == MODE_MAIN && st_n > kStageCap - kStageBurst) flush();
      const bool more0 = qf + 1 < nqf;
      if (more0) {
        mfmas(c1, a, sa, b1, qf + 1);
        tc1 = t1;
        load_b(b0, t0, min(qf + 2, nqf - 1));
      }
      if (MODE == MODE_SAMPLE) {
        epi_sample(c0, wd, f0, qf);
      } else {
        epi_fast(c0, tc0, hit);
        epi_slow(c0, hit, f0, qf, tc0);
      }
      if (!more0) break;
      ++qf;
      // c1 holds fragment qf; b0 holds fragment qf+1's operand.
      if (MODE == MODE_MAIN && st_n > kStageCap - kStageBurst) flush();
      const bool more1 = qf + 1 < nqf;
      if (more1) {
        mfmas(c0, a, sa, b0, qf + 1);
        tc0 = t0;
        load_b(b1, t1, min(qf + 2, nqf - 1));
      }
      if (MODE == MODE_SAMPLE) {
        epi_sample(c1, wd, f0, qf);
      } else {
        epi_fast(c1, tc1, hit);
        epi_slow(c1, hit, f0, qf, tc1);
      }
      if (!more1) break;
      ++qf;
    }
  };

  const int64_t t_begin = (int64_t)slice * A.ntiles / A.nslices;
  const int64_t t_end = (int64_t)(slice + 1) * A.ntiles / A.nslices;

  // Two-stage software pipeline: the next stage's corpus fragments are in flight while
  // the current stage is multiplied against every query fragment.
  u32x4_t a0[RM][NCH], a1[RM][NCH];
  int s0[RM], s1[RM];
  uint32_t w0[RM], w1[RM];
  int64_t t = t_begin + wave;
  if (t < t_end) {
    // Threshold refreshes are committed one stage after they are issued: they were issued
    // before that stage's corpus loads, so waiting for them then is free.
    if (MODE == MODE_MAIN) refresh_issue();
    load_stage(a0, s0, w0, t * RM);
    for (;;) {
      const int64_t t1 = t + kScoreWaves;
      if (MODE == MODE_MAIN) {
        refresh_commit();
        refresh_issue();
      }
      load_stage(a1, s1, w1, t1 * RM);
      compute_stage(a0, s0, w0, t * RM);
      if (t1 >= t_end) break;
      const int64_t t2 = t1 + kScoreWaves;
      if (MODE == MODE_MAIN) {
        refresh_commit();
        refresh_issue();
      }
      load_stage(a0, s0, w0, t2 * RM);
      compute_stage(a1, s1, w1, t1 * RM);
      if (t2 >= t_end) break;
      t = t2;
    }
  }
  if (MODE == MODE_MAIN && st_n > 0) flush();
}

// ------------------------------------------------------------------ query prep
template <int CT, int QT, int D>
__global__ __launch_bounds__(64) void prep_queries_kernel(const void* __restrict__ queries, int b,
                                                          uint8_t* __restrict__ qtile,
                                                          int* __restrict__ qexp,
                                                          uint32_t* __restrict__ thr,
                                                          uint32_t* __restrict__ cnt,
                                                          uint32_t* __restrict__ ovf,
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
    ovf[q] = 0u;
    for (int j = 0; j < kLevels; ++j) {
      lvl[(int64_t)q * kLevels + j] = 0xFFFFFFFFu;
      lcnt[(int64_t)q * kLevels + j] = 0u;
    }
  }
}

// --------------------------------------------------------------- radix select
// Block-wide helpers; every caller runs with kSelThreads (= 256) threads.

struct DigitPick {
  uint32_t digit, rem, bin;
};

// hist[0..255]: keys per digit value (under the current prefix). Finds the digit d with
// fewer than `rem` keys above it and at least `rem` at or above it, by a prefix sum over
// the bins taken from the top. Returns d, the rank left inside bin d and the bin's size.
__device__ DigitPick pick_digit(const uint32_t* hist, uint32_t rem, uint32_t* wsum,
                                DigitPick* out) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint32_t h = hist[255 - t];
  uint32_t c = h;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_up(c, o, kWave);
    if (lane >= o) c += u;
  }
  if (lane == kWave - 1) wsum[w] = c;
  __syncthreads();
  for (int i = 0; i < w; ++i) c += wsum[i];
  const uint32_t prev = c - h;
  if (prev < rem && c >= rem) *out = DigitPick{(uint32_t)(255 - t), rem - prev, h};
  __syncthreads();
  const DigitPick r = *out;
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Selection state: the keys with (key & mask) >= prefix are the r largest.
struct Sel64 {
  uint64_t prefix, mask;
};

struct SelScratch {
  uint32_t hist[256];
  uint32_t wsum[4];
  DigitPick pick;
  uint64_t red[8];
};

// The r largest of n keys (1 <= r <= n), MSD radix select with 8-bit digits starting at
// the highest bit where the keys differ; stops as soon as the boundary bin holds exactly
// the remaining rank. With distinct keys exactly r keys satisfy the returned test; with
// ties, prefix is still a lower bound of the r-th largest key.
template <typename Get>
__device__ Sel64 select_top(Get get, int64_t n, int r, SelScratch& S) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint64_t lo = ~0ull, hi = 0ull;
  for (int64_t i = t; i < n; i += kSelThreads) {
    const uint64_t k = get(i);
    lo = k < lo ? k : lo;
    hi = k > hi ? k : hi;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t l2 = shfl_xor_u64(lo, o), h2 = shfl_xor_u64(hi, o);
    lo = l2 < lo ? l2 : lo;
    hi = h2 > hi ? h2 : hi;
  }
  if (lane == 0) {
    S.red[w] = lo;
    S.red[4 + w] = hi;
  }
  __syncthreads();
  lo = S.red[0];
  hi = S.red[4];
  for (int i = 1; i < 4; ++i) {
    lo = S.red[i] < lo ? S.red[i] : lo;
    hi = S.red[4 + i] > hi ? S.red[4 + i] : hi;
  }
  __syncthreads();
  const uint64_t diff = lo ^ hi;
  if (diff == 0ull) return Sel64{lo, ~0ull};  // all keys equal
  int hb = 63 - __builtin_clzll(diff);        // highest bit not yet fixed
  uint64_t mask = hb == 63 ? 0ull : ~((2ull << hb) - 1ull);
  uint64_t prefix = lo & mask;
  uint32_t rem = (uint32_t)r;
  for (;;) {
    const int lb = hb >= 7 ? hb - 7 : 0;
    const int width = hb - lb + 1;
    const uint64_t dmask = (1ull << width) - 1ull;
    S.hist[t] = 0u;
    __syncthreads();
    for (int64_t i = t; i < n; i += kSelThreads) {
      const uint64_t k = get(i);
      if ((k & mask) == prefix) atomicAdd(&S.hist[(k >> lb) & dmask], 1u);
    }
    __syncthreads();
    const DigitPick pk = pick_digit(S.hist, rem, S.wsum, &S.pick);
    prefix |= (uint64_t)pk.digit << lb;
    mask |= dmask << lb;
    rem = pk.rem;
    if (pk.bin == pk.rem || lb == 0) break;
    hb = lb - 1;
  }
  return Sel64{prefix, mask};
}

// Descending bitonic sort of p (a power of two) 64-bit keys in LDS.
__device__ void bitonic_desc(uint64_t* s, int p) {
  for (int size = 2; size <= p; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (p >> 1); i += kSelThreads) {
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

__device__ __forceinline__ int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Per query: the K-th largest delegate is the starting threshold (K distinct blocks hold an
// item at least that good). The delegates of geometrically spaced ranks below K become the
// levels: once K survivors reach a level, the level is a valid threshold too.
__global__ __launch_bounds__(kSelThreads) void sample_threshold_kernel(const uint32_t* __restrict__ del,
                                                                       int G, int b, int k,
                                                                       float rank_ratio,
                                                                       uint32_t* __restrict__ thr,
                                                                       uint32_t* __restrict__ lvl) {
  __shared__ uint32_t keys[kSampleGroups];
  __shared__ uint64_t top[2048];
  __shared__ SelScratch S;
  __shared__ uint32_t ntop;
  const int q = blockIdx.x;
  if (q >= b) return;
  for (int i = threadIdx.x; i < G; i += kSelThreads) keys[i] = del[(int64_t)q * G + i];
  if (threadIdx.x == 0) ntop = 0u;
  __syncthreads();
  uint32_t kth = 0u;
  if (G >= k) {
    const Sel64 sel = select_top([&](int64_t i) { return (uint64_t)keys[i]; }, G, k, S);
    kth = (uint32_t)sel.prefix;
  }
  for (int i = threadIdx.x; i < G; i += kSelThreads) {
    if (keys[i] >= kth && keys[i] != 0u) {
      const uint32_t slot = atomicAdd(&ntop, 1u);
      if (slot < 2048u) top[slot] = keys[i];
    }
  }
  __syncthreads();
  const int m = (int)min(ntop, 2048u);
  const int p = pow2_at_least(m < 2 ? 2 : m);
  for (int i = m + threadIdx.x; i < p; i += kSelThreads) top[i] = 0u;
  __syncthreads();
  bitonic_desc(top, p);
  if (threadIdx.x < kLevels) {
    // Level j sits at sample rank k * rho^(j+1), rho chosen so the last level lands near
    // the sample rank the final K-th best is expected at (k / rank_ratio).
    const int j = threadIdx.x;
    const float rmin = fmaxf(1.0f, 0.5f * (float)k / rank_ratio);
    const float rho = powf(rmin / (float)k, 1.0f / (float)kLevels);
    const int rank = (int)ceilf((float)k * powf(rho, (float)(j + 1)));
    uint32_t v = 0xFFFFFFFFu;
    if (rank >= 1 && rank < k && rank <= m) v = (uint32_t)top[rank - 1];
    if (v == 0u) v = 0xFFFFFFFFu;
    lvl[(int64_t)q * kLevels + j] = v;
  }
  if (threadIdx.x == 0) thr[q] = kth;
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
  const uint32_t* ovf;
  const uint64_t* cand;
  float* out_scores;
  int32_t* out_ids;
};

constexpr int kSelCache = 6144;  // candidates cached in LDS by the final select

// Writes query q's sorted keys (descending) and pads the rest with (-inf, -1).
__device__ void write_out(const SelectArgs& A, int q, const uint64_t* s, int cnt) {
  for (int t = threadIdx.x; t < A.k; t += kSelThreads) {
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

// Gathers the r selected keys of `get` into out[0..r), sorts them descending.
template <typename Get>
__device__ void gather_sort(Get get, int64_t n, int r, Sel64 sel, uint64_t* out, uint32_t* cnt) {
  if (threadIdx.x == 0) *cnt = 0u;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < n; i += kSelThreads) {
    const uint64_t key = get(i);
    if ((key & sel.mask) >= sel.prefix) {
      const uint32_t slot = atomicAdd(cnt, 1u);
      if (slot < (uint32_t)r) out[slot] = key;
    }
  }
  __syncthreads();
  const int p = pow2_at_least(r < 2 ? 2 : r);
  for (int i = r + threadIdx.x; i < p; i += kSelThreads) out[i] = 0u;
  __syncthreads();
  bitonic_desc(out, p);
}

// Exact rescan of query q: VALU dot products in dimension order, candidates buffered in
// LDS behind a composite-key threshold that rises whenever the buffer is compacted to
// its k best.
template <int CT, int D>
__device__ void fallback_scan(const SelectArgs& A, int q, uint64_t thr, uint64_t* buf,
                              uint64_t* sel_buf, SelScratch& S, float* qv, uint32_t* nbuf_p) {
  for (int j = threadIdx.x; j < D; j += kSelThreads) {
    const int64_t off = (int64_t)(q >> 5) * block_bytes(CT, D) + packed_offset(CT, D, q & 31, j);
    float v;
    if (CT == MIPS_F32)
      v = *(const float*)(A.qtile + off);
    else if (CT == MIPS_BF16)
      v = bf16_to_f32(*(const uint16_t*)(A.qtile + off));
    else
      v = e4m3_to_f32(A.qtile[off]) * exp2_int(A.qexp[q] - 127);
    qv[j] = v;
  }
  if (threadIdx.x == 0) *nbuf_p = 0u;
  __syncthreads();
  constexpr int kRound = kSelThreads * 4;
  for (int64_t base = 0; base < A.n; base += kRound) {
    if (*nbuf_p + (uint32_t)kRound > (uint32_t)kSelCache) {
      // Compact to the k best and raise the threshold to their lower bound.
      const int m = (int)*nbuf_p;
      const int r = min(A.k, m);
      const Sel64 sel = select_top([&](int64_t i) { return buf[i]; }, m, r, S);
      gather_sort([&](int64_t i) { return buf[i]; }, m, r, sel, sel_buf, &S.hist[0]);
      for (int i = threadIdx.x; i < r; i += kSelThreads) buf[i] = sel_buf[i];
      if (threadIdx.x == 0) *nbuf_p = (uint32_t)r;
      if (r == A.k) thr = sel_buf[r - 1] > thr ? sel_buf[r - 1] : thr;
      __syncthreads();
    }
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + (int64_t)u * kSelThreads + threadIdx.x;
      if (i >= A.n || is_excluded(A.exclude, i)) continue;
      float s = 0.0f;
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
      if (CT == MIPS_FP8_E4M3) s *= A.row_scale[i];
      const uint64_t key = composite(score_key(s), (uint32_t)i);
      if (key >= thr) buf[atomicAdd(nbuf_p, 1u)] = key;
    }
    __syncthreads();
  }
  const int m = (int)*nbuf_p;
  const int r = min(A.k, m);
  if (r > 0) {
    Sel64 sel{0ull, 0ull};
    if (m > r) sel = select_top([&](int64_t i) { return buf[i]; }, m, r, S);
    gather_sort([&](int64_t i) { return buf[i]; }, m, r, sel, sel_buf, &S.hist[0]);
  }
  write_out(A, q, sel_buf, r);
}

template <int CT, int D>
__global__ __launch_bounds__(kSelThreads) void final_select_kernel(SelectArgs A) {
  __shared__ uint64_t cache[kSelCache];
  __shared__ uint64_t sel_buf[MIPS_K_MAX];
  __shared__ SelScratch S;
  __shared__ float qv[D];
  __shared__ uint32_t nbuf;
  const int q = blockIdx.x;
  if (q >= A.b) return;
  const int64_t c = A.cnt[q];
  const uint64_t* list = A.cand + (int64_t)q * A.cap;
  if (c > A.cap || A.ovf[q] != 0u) {
    // The list is incomplete. Its stored entries are still real candidates, so their
    // k-th best bounds the exact rescan from below.
    uint64_t start = 0ull;
    const int64_t stored = min<int64_t>(c, A.cap);
    if (stored >= A.k) start = select_top([&](int64_t i) { return list[i]; }, stored, A.k, S).prefix;
    __syncthreads();
    fallback_scan<CT, D>(A, q, start, cache, sel_buf, S, qv, &nbuf);
    return;
  }
  const int r = (int)min<int64_t>(c, A.k);
  if (r > 0) {
    if (c <= kSelCache) {
      for (int64_t i = threadIdx.x; i < c; i += kSelThreads) cache[i] = list[i];
      __syncthreads();
      auto get = [&](int64_t i) { return cache[i]; };
      Sel64 sel{0ull, 0ull};
      if (c > r) sel = select_top(get, c, r, S);
      gather_sort(get, c, r, sel, sel_buf, &S.hist[0]);
    } else {
      auto get = [&](int64_t i) { return list[i]; };
      const Sel64 sel = select_top(get, c, r, S);
      gather_sort(get, c, r, sel, sel_buf, &S.hist[0]);
    }
  }
  write_out(A, q, sel_buf, r);
}

// ------------------------------------------------------------------- planning
struct Plan {
  int b, b32, k, d, qdt, cdt;
  int64_t n, n32;
  int rm, qb, nqblk, G;
  int64_t ntiles, cap;
  size_t off_qtile, off_qexp, off_thr, off_cnt, off_ovf, off_lvl, off_lcnt, off_del, off_cand, fixed;
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
  p.rm = stage_frags(cdt, d);
  p.ntiles = (p.n32 + p.rm - 1) / p.rm;
  const int E = elem_bytes(cdt);
  // LDS per query: its operand row, its fp8 exponent, its threshold and its levels; plus
  // each wave's survivor staging buffer.
  const int stage_bytes = kScoreWaves * kStageCap * 10;
  const int per_query = d * E + 4 + 4 + 4 * kLevels;
  int qb = (kLdsScoreBudget - stage_bytes) / per_query;
  qb = qb / 32 * 32;
  if (qb > kMaxQueryBlock) qb = kMaxQueryBlock;
  if (qb > p.b32) qb = p.b32;
  p.nqblk = (p.b32 + qb - 1) / qb;
  p.qb = ((p.b32 + p.nqblk - 1) / p.nqblk + 31) / 32 * 32;
  p.lds_score = (size_t)p.qb * per_query + (size_t)stage_bytes;
  size_t o = 0;
  p.off_qtile = o;
  o = align256(o + (size_t)p.b32 * d * E);
  p.off_qexp = o;
  o = align256(o + (size_t)p.b32 * 4);
  p.off_thr = o;
  o = align256(o + (size_t)b * 4);
  p.off_cnt = o;
  o = align256(o + (size_t)b * 4);
  p.off_ovf = o;
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
  uint32_t* ovf = (uint32_t*)(ws + p.off_ovf);
  uint32_t* lvl = (uint32_t*)(ws + p.off_lvl);
  uint32_t* lcnt = (uint32_t*)(ws + p.off_lcnt);
  uint32_t* del = (uint32_t*)(ws + p.off_del);
  uint64_t* cand = (uint64_t*)(ws + p.off_cand);

  if (p.qdt == MIPS_F32)
    hipLaunchKernelGGL((prep_queries_kernel<CT, MIPS_F32, D>), dim3(p.b32 / 32), dim3(64), 0, s,
                       queries, p.b, qtile, qexp, thr, cnt, ovf, lvl, lcnt);
  else
    hipLaunchKernelGGL((prep_queries_kernel<CT, MIPS_BF16, D>), dim3(p.b32 / 32), dim3(64), 0, s,
                       queries, p.b, qtile, qexp, thr, cnt, ovf, lvl, lcnt);
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
  A.ovf = ovf;
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
                       p.k, (float)((double)p.n32 / (double)p.G), thr, lvl);
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
  S.ovf = ovf;
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
    case 256: if constexpr (CT != MIPS_F32) { MIPS_RUN(256); } break;
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
