// score.h -- the fused MFMA score pass of mips_topk for gfx950 (sample, dense and main
// epilogues); included only by score_inst.hip.
#pragma once

#include "host.h"
#include "score_api.h"

namespace mips {

template <int CT>
__device__ __forceinline__ void mfma_step(f32x16_t& acc, const u32x4_t* a, const u32x4_t* b,
                                          int sa, int sb, int s) {
  if constexpr (CT == MIPS_BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[s]),
                                                  __builtin_bit_cast(bf16x8_t, b[s]), acc, 0, 0, 0);
  } else if constexpr (CT == MIPS_FP8_E4M3) {
    i32x8_t av, bv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      av[j] = (int)a[2 * s][j];
      av[4 + j] = (int)a[2 * s + 1][j];
      bv[j] = (int)b[2 * s][j];
      bv[4 + j] = (int)b[2 * s + 1][j];
    }
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, sa, 0, sb);
  } else {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[s >> 2][s & 3]),
                                               __uint_as_float(b[s >> 2][s & 3]), acc, 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t lane_rank(uint64_t bm) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
}

// One workgroup = 4 waves (one per SIMD) = one corpus slice x one block of 32 * NQF
// queries. Each wave streams stage tiles of RM 32-row blocks (16 KiB) into registers, two
// stages in flight, and multiplies each stage against every query fragment of the block
// in LDS. The query-fragment loop is unrolled and software-pipelined: the MFMAs of
// fragment qf+1 and the LDS reads of fragment qf+2's operand are issued before the
// epilogue of fragment qf.
template <int CT, int D, int NQF, int MODE>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs A) {
  constexpr int E = elem_bytes(CT);
  constexpr int NCH = chunks_per_block(CT, D);
  constexpr int RM = stage_frags(CT, D);
  constexpr int KSTEPS = (CT == MIPS_F32) ? D / 2 : (CT == MIPS_BF16 ? D / 16 : D / 64);
  constexpr int64_t BLK = block_bytes(CT, D);
  constexpr int QB = kFrag * NQF;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool rescue = A.nlist != nullptr;

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

  // LDS: query operand tile | global query id per column | per-wave survivor staging
  // (composite keys, query column).
  int* qid_lds = (int*)(lds + (size_t)QB * D * E);
  uint64_t* st_key = (uint64_t*)(qid_lds + QB) + wave * kStageCap;
  uint16_t* st_q = (uint16_t*)((uint64_t*)(qid_lds + QB) + kScoreWaves * kStageCap) + wave * kStageCap;

  const int64_t t_begin = (int64_t)slice * A.ntiles / A.nslices;
  const int64_t t_end = (int64_t)(slice + 1) * A.ntiles / A.nslices;
  const int nq_total = rescue ? (int)*A.nlist : A.b;
  const int qstep = rescue ? 1 : A.nqblk;

  for (int qb = rescue ? 0 : qblk; qb * QB < nq_total; qb += qstep) {
    const int qbase = qb * QB;
    __syncthreads();
    if (!rescue) {
      const int rows = min(QB, A.b32 - qbase);
      const u32x4_t* src = (const u32x4_t*)(A.qtile + (int64_t)qbase * D * E);
      u32x4_t* dst = (u32x4_t*)lds;
      const int n16 = rows * D * E / 16;
      for (int i = threadIdx.x; i < QB * D * E / 16; i += kScoreThreads)
        dst[i] = i < n16 ? src[i] : u32x4_t{0u, 0u, 0u, 0u};
      for (int i = threadIdx.x; i < QB; i += kScoreThreads) qid_lds[i] = qbase + i < A.b ? qbase + i : -1;
    } else {
      for (int i = threadIdx.x; i < QB; i += kScoreThreads)
        qid_lds[i] = qbase + i < nq_total ? (int)A.qlist[qbase + i] : -1;
      __syncthreads();
      // gather the queued queries' operand rows: 16-byte slot s of chunk c of column
      // fragment qf comes from slot (q & 31) + 32 (s >> 5) of the same chunk of q's block
      u32x4_t* dst = (u32x4_t*)lds;
      for (int i = threadIdx.x; i < QB * D * E / 16; i += kScoreThreads) {
        const int s = i & 63, c = (i >> 6) % NCH, qf = (i >> 6) / NCH;
        const int q = qid_lds[qf * kFrag + (s & 31)];
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (q >= 0)
          v = *(const u32x4_t*)(A.qtile + (int64_t)(q >> 5) * BLK + c * kChunkBytes +
                                ((q & 31) + 32 * (s >> 5)) * 16);
        dst[i] = v;
      }
    }
    __syncthreads();

    // This lane's query column in each fragment: threshold, fp8 exponent, global id.
    float Tq[NQF];
    int sbq[NQF], qgq[NQF];
#pragma unroll
    for (int qf = 0; qf < NQF; ++qf) {
      const int qg = qid_lds[qf * kFrag + (lane & 31)];
      qgq[qf] = qg;
      float T = INFINITY;
      if (MODE == MODE_MAIN && qg >= 0) {
        const uint32_t k = A.thr[qg];
        if (k != 0u) T = key_threshold(k);
      }
      Tq[qf] = T;
      sbq[qf] = (CT == MIPS_FP8_E4M3 && qg >= 0) ? A.qexp[qg] : 127;
    }

    int st_n = 0;  // staged survivors of this wave (wave-uniform; may exceed the capacity)

    // Appends the staged survivors to their queries' lists: all returning atomics are
    // issued before the first store waits for one.
    auto flush = [&]() {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int nst = min(st_n, kStageCap);
      constexpr int R = kStageCap / kWave;
      uint64_t ck[R];
      uint32_t pos[R];
      int qg[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int e = r * kWave + lane;
        ck[r] = 0ull;
        qg[r] = 0;
        pos[r] = 0xFFFFFFFFu;
        if (e < nst) {
          ck[r] = st_key[e];
          qg[r] = qid_lds[st_q[e]];
          pos[r] = atomicAdd(&A.cnt[qg[r]], 1u);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
        if ((int64_t)pos[r] < A.cap) A.cand[(int64_t)qg[r] * A.cap + pos[r]] = ck[r];
      __builtin_amdgcn_wave_barrier();
      st_n = 0;
    };

    // A stage's loads are unconditional: blocks past the end of the pass read the last
    // block again and are masked out, so the compiler's wait counts stay exact. Lane r < RM
    // also loads the exclusion word of block r, with the rows past n set.
    auto load_stage = [&](u32x4_t (&a)[RM][NCH], int (&sa)[RM], uint32_t& xwv, int64_t j0) {
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        const int64_t j = min<int64_t>(j0 + r, A.nfrag - 1);
        const int64_t fr = (MODE == MODE_AUX && !A.dense) ? j * A.n32 / A.nfrag : j;
        const u32x4_t* p = (const u32x4_t*)(A.corpus + fr * BLK) + lane;
#pragma unroll
        for (int c = 0; c < NCH; ++c) a[r][c] = p[c * (kChunkBytes / 16)];
        sa[r] = 127;
        if (CT == MIPS_FP8_E4M3)
          sa[r] = (int)((__float_as_uint(A.row_scale[fr * kFrag + (lane & 31)]) >> 23) & 0xFFu);
      }
      const int r = lane < RM ? lane : RM - 1;
      const bool live = j0 + r < A.nfrag;
      const int64_t j = live ? j0 + r : A.nfrag - 1;
      const int64_t fr = (MODE == MODE_AUX && !A.dense) ? j * A.n32 / A.nfrag : j;
      uint32_t w = A.exclude ? A.exclude[fr] : 0u;
      const int64_t rows = A.n - fr * kFrag;
      if (rows < kFrag) w |= ~0u << rows;
      xwv = live ? w : ~0u;
    };

    auto load_b = [&](u32x4_t (&bq)[NCH], int qf) {
      const u32x4_t* bsrc = (const u32x4_t*)(lds + (size_t)qf * BLK) + lane;
#pragma unroll
      for (int c = 0; c < NCH; ++c) bq[c] = bsrc[c * (kChunkBytes / 16)];
    };
    auto mfmas = [&](f32x16_t (&acc)[RM], const u32x4_t (&a)[RM][NCH], const int (&sa)[RM],
                     const u32x4_t (&bq)[NCH], int sb) {
#pragma unroll
      for (int g = 0; g < RM; ++g) acc[g] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int g = 0; g < RM; ++g) mfma_step<CT>(acc[g], a[g], bq, sa[g], sb, s);
    };

    // Main epilogue of one query fragment: one max per block (16 scores per lane) and one
    // ballot, branch-free so it interleaves with the next fragment's MFMAs. A block that
    // clears the threshold is resolved by 4-row groups, then value by value with ballot +
    // mbcnt compaction into the wave's staging buffer; those loops index the accumulators
    // with a wave-uniform runtime index and stay rolled.
    auto epi_main = [&](const f32x16_t (&acc)[RM], uint32_t xwv, int64_t j0, int qf) {
      const float T = Tq[qf];
      float m[RM];
      bool any = false;
#pragma unroll
      for (int g = 0; g < RM; ++g) {
        float x = acc[g][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) x = fmaxf(x, acc[g][i]);
        m[g] = x;
        any = any || (x >= T);
      }
      if (__builtin_expect(__ballot(any) != 0ull, 0)) {
        const int ql = qf * kFrag + (lane & 31);
#pragma unroll
        for (int g = 0; g < RM; ++g) {
          if (__ballot(m[g] >= T) == 0ull) continue;
          const uint32_t w = __builtin_amdgcn_readlane(xwv, g);
          const uint32_t idb = (uint32_t)((j0 + g) * kFrag);
#pragma unroll 1
          for (int bb = 0; bb < 4; ++bb) {
            const float pm = fmaxf(fmaxf(acc[g][4 * bb], acc[g][4 * bb + 1]),
                                   fmaxf(acc[g][4 * bb + 2], acc[g][4 * bb + 3]));
            if (__ballot(pm >= T) == 0ull) continue;
#pragma unroll 1
            for (int i = 4 * bb; i < 4 * bb + 4; ++i) {
              const float v = acc[g][i];
              const int row = acc_row(i, lane);
              const bool pass = v >= T && !((w >> row) & 1u);
              const uint64_t bm = __ballot(pass);
              if (bm == 0ull) continue;
              const int pos = st_n + (int)lane_rank(bm);
              if (pass) {
                if (pos < kStageCap) {
                  st_key[pos] = composite(score_key(v), idb + (uint32_t)row);
                  st_q[pos] = (uint16_t)ql;
                } else {
                  atomicOr(&A.ovf[qid_lds[ql]], 1u);  // no room: the query is rescued
                }
              }
              st_n += __popcll(bm);
            }
          }
        }
      }
    };

    // Auxiliary epilogue. Dense pass: every score of the block goes to the query's list at
    // its id (0 for excluded and padding rows). Sample pass: the best eligible score of the
    // block is the (block, query) delegate (key 0 if the block has no eligible row).
    auto epi_aux = [&](const f32x16_t (&acc)[RM], uint32_t xwv, int64_t j0, int qf) {
      const int qg = qgq[qf];
#pragma unroll
      for (int g = 0; g < RM; ++g) {
        const int64_t j = j0 + g;
        const uint32_t w = __builtin_amdgcn_readlane(xwv, g);
        if (A.dense) {
          if (j < A.nfrag && qg >= 0) {
            uint64_t* dst = A.cand + (int64_t)qg * A.cap + j * kFrag;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int row = acc_row(i, lane);
              dst[row] = ((w >> row) & 1u) ? 0ull
                                           : composite(score_key(acc[g][i]), (uint32_t)(j * kFrag + row));
            }
          }
        } else {
          float mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = acc_row(i, lane);
            mx = ((w >> row) & 1u) ? mx : fmaxf(mx, acc[g][i]);
          }
          mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
          const int qc = qbase + qf * kFrag + lane;
          if (lane < kFrag && j < A.nfrag && qc < A.b32)
            A.del[j * A.b32 + qc] = (mx == -INFINITY) ? 0u : score_key(mx);
        }
      }
    };

    auto compute_stage = [&](const u32x4_t (&a)[RM][NCH], const int (&sa)[RM], uint32_t xwv,
                             int64_t j0) {
      u32x4_t bq[2][NCH];
      f32x16_t acc[2][RM];
      load_b(bq[0], 0);
      if (NQF > 1) load_b(bq[1], 1);
      mfmas(acc[0], a, sa, bq[0], sbq[0]);
#pragma unroll
      for (int qf = 0; qf < NQF; ++qf) {
        const int cur = qf & 1;
        if (qf + 1 < NQF) {
          mfmas(acc[cur ^ 1], a, sa, bq[cur ^ 1], sbq[qf + 1 < NQF ? qf + 1 : 0]);
          if (qf + 2 < NQF) load_b(bq[cur], qf + 2 < NQF ? qf + 2 : 0);
        }
        if (MODE == MODE_MAIN)
          epi_main(acc[cur], xwv, j0, qf);
        else
          epi_aux(acc[cur], xwv, j0, qf);
      }
    };

    // Two-stage software pipeline over this wave's stage tiles: the next stage's corpus
    // blocks are in flight while the current one is multiplied against every query.
    u32x4_t a0[RM][NCH], a1[RM][NCH];
    int s0[RM], s1[RM];
    uint32_t x0, x1;
    int64_t t = t_begin + wave;
    if (t < t_end) {
      load_stage(a0, s0, x0, t * RM);
      for (;;) {
        const int64_t t1 = t + kScoreWaves;
        load_stage(a1, s1, x1, t1 < t_end ? t1 * RM : A.nfrag);
        if (MODE == MODE_MAIN && st_n > kStageCap - kStageBurst) flush();
        compute_stage(a0, s0, x0, t * RM);
        if (t1 >= t_end) break;
        const int64_t t2 = t1 + kScoreWaves;
        load_stage(a0, s0, x0, t2 < t_end ? t2 * RM : A.nfrag);
        if (MODE == MODE_MAIN && st_n > kStageCap - kStageBurst) flush();
        compute_stage(a1, s1, x1, t1 * RM);
        if (t2 >= t_end) break;
        t = t2;
      }
    }
    if (MODE == MODE_MAIN && st_n > 0) flush();
  }
}

template <int CT, int D, int NQF, int MODE>
static int launch_score(const ScoreArgs& A, int grid, hipStream_t s) {
  constexpr int lds = score_lds_bytes(CT, D, NQF);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)score_kernel<CT, D, NQF, MODE>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  hipLaunchKernelGGL((score_kernel<CT, D, NQF, MODE>), dim3(grid), dim3(kScoreThreads), lds, s, A);
  return check_launch();
}

template <int CT, int D, int MODE>
int launch_score_nqf(int nqf, const ScoreArgs& A, int grid, hipStream_t s) {
  switch (nqf) {
    case 1: return launch_score<CT, D, 1, MODE>(A, grid, s);
    case 2: return launch_score<CT, D, 2, MODE>(A, grid, s);
    case 4: return launch_score<CT, D, 4, MODE>(A, grid, s);
    case 8:
      if constexpr (nqf_fits(CT, D, 8)) return launch_score<CT, D, 8, MODE>(A, grid, s);
      break;
    case 16:
      if constexpr (nqf_fits(CT, D, 16)) return launch_score<CT, D, 16, MODE>(A, grid, s);
      break;
  }
  return MIPS_ERR_UNSUPPORTED;
}

}  // namespace mips
