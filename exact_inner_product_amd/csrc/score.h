// score.h -- the fused MFMA score pass of mips_topk for gfx950 (sample, dense and main
// epilogues); included only by score_inst.hip.
#pragma once

#include <utility>

#include <hip/hip_ext.h>

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
  } else if constexpr (CT == MIPS_INT8) {
    // int32 accumulation; the accumulator registers hold the integer bits
    acc = __builtin_bit_cast(
        f32x16_t, __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, a[s]),
                                                        __builtin_bit_cast(i32x4_t, b[s]),
                                                        __builtin_bit_cast(i32x16_t, acc), 0, 0, 0));
  } else {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[s >> 2][s & 3]),
                                               __uint_as_float(b[s >> 2][s & 3]), acc, 0, 0, 0);
  }
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time (the
// register arrays it indexes must never be indexed at run time).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Buffer descriptor of `bytes` bytes at p (gfx9 raw buffer: stride 0, offsets in bytes;
// loads past the range return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// One workgroup = 4 or 8 waves (one or two per SIMD) = one corpus slice x one block of
// 32 * NQF queries. Each wave streams stage tiles of RM 32-row blocks (16 KiB per SIMD)
// into registers, two stages in flight, and multiplies each stage against every query
// fragment of the block in LDS. The query-fragment loop is unrolled and software-pipelined:
// the MFMAs of fragment qf+1 and the LDS reads of fragment qf+2's operand are issued
// before the epilogue of fragment qf. With NT > 0 (a multi-mask pass) every score is
// tested against up to NT masks, each with its own threshold and list per query.
template <int CT, int D, int NQF, int MODE, int NT>
__global__ __launch_bounds__(score_threads(CT, D))
__attribute__((amdgpu_waves_per_eu(score_wps(CT, D), score_wps(CT, D)))) void score_kernel(ScoreArgs A) {
  constexpr int kScoreThreads = score_threads(CT, D);
  constexpr int kScoreWaves = score_waves(CT, D);
  constexpr int E = elem_bytes(CT);
  constexpr int NCH = chunks_per_block(CT, D);
  constexpr int RM = MODE == MODE_MAIN ? main_frags(CT, D) : stage_frags(CT, D);
  constexpr bool SINGLE = MODE == MODE_MAIN && main_doubles(CT, D);  // one accumulator set
  constexpr int KSTEPS = (CT == MIPS_F32) ? D / 2
                        : (CT == MIPS_BF16 ? D / 16 : (CT == MIPS_INT8 ? D / 32 : D / 64));
  // int8: per stage block, the scales of the 16 rows a lane's accumulators cover
  constexpr int SCN = CT == MIPS_INT8 ? 16 : 1;
  constexpr int64_t BLK = block_bytes(CT, D);
  constexpr int QB = kFrag * NQF;
  constexpr int NTS = NT > 0 ? NT : 1;  // survivor counters per query column
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

  // LDS: query operand tile | per column: global query id, segment counter(s), threshold,
  // fp8 exponent or int8 scale | multi-mask: threshold per column and mask | per-wave
  // survivor staging (composite keys, query column; column * NT + mask with masks).
  int* qid_lds = (int*)(lds + (size_t)QB * D * E);
  uint32_t* seg_lds = (uint32_t*)(qid_lds + QB);  // survivors per query column (and mask)
  float* thr_lds = (float*)(seg_lds + QB * NTS);  // threshold per query column (lowest mask's)
  int* sexp_lds = (int*)(thr_lds + QB);           // fp8 exponent / int8 scale per column
  float* thrt_lds = (float*)(sexp_lds + QB);      // [QB][NT] thresholds of a multi-mask pass
  uint64_t* st_key = (uint64_t*)(sexp_lds + QB + QB * NT) + wave * kStageCap;
  uint16_t* st_q = (uint16_t*)((uint64_t*)(sexp_lds + QB + QB * NT) + kScoreWaves * kStageCap) + wave * kStageCap;

  // The corpus slices' shares of the tiles. With the slices spread over the 8 XCDs (slice s on
  // XCD s % 8, the dispatch order), an odd XCD's slice takes 24 shares to an even XCD's 25:
  // timed per workgroup, the odd XCDs ran 2-5% slower than the even ones (a lower shader
  // clock) on every call, so that the pass ended with them.
  int64_t t_begin, t_end;
  if (A.nslices % 8 == 0) {
    auto cum = [](int64_t s) { return (s >> 1) * 49 + (s & 1) * 25; };
    const int64_t W = cum(A.nslices);
    t_begin = A.ntiles * cum(slice) / W;
    t_end = A.ntiles * cum(slice + 1) / W;
  } else {
    t_begin = (int64_t)slice * A.ntiles / A.nslices;
    t_end = (int64_t)(slice + 1) * A.ntiles / A.nslices;
  }
  const int nq_total = rescue ? (int)*A.nlist : A.b;
  const int qstep = rescue ? 1 : A.nqblk;

  for (int qb = rescue ? 0 : qblk; qb * QB < nq_total; qb += qstep) {
    const int qbase = qb * QB;
    __syncthreads();
    // The query tile is NV 16-byte units; each thread moves PER of them, kFillBatch loads
    // in flight per round trip.
    constexpr int NV = QB * D * E / 16;
    constexpr int kFillBatch = 4;
    constexpr int PER = (NV + kScoreThreads - 1) / kScoreThreads;
    if (fused_prep_ok(CT, D, NQF) && MODE == MODE_SAMPLE && !rescue && A.qraw != nullptr) {
      // the operand tile from the raw queries (the layout of the packed corpus, 32 queries
      // per block); rounding as the query prep kernel's
      const int rows = min(QB, A.b32 - qbase);
      const int n16 = rows * D * E / 16;
      u32x4_t* dst = (u32x4_t*)lds;
      u32x4_t* gdst = (u32x4_t*)(const_cast<uint8_t*>(A.qtile) + (int64_t)qbase * D * E);
      // slot s of chunk c: bf16 dims 16c + 8h + (0..7), contiguous; f32 dims 8c + h + 2t
      constexpr int kRawBatch = 8;
      for (int i0 = 0; i0 < PER; i0 += kRawBatch) {
        u32x4_t v[kRawBatch];
#pragma unroll
        for (int u = 0; u < kRawBatch; ++u) {
          const int i = (i0 + u) * kScoreThreads + threadIdx.x;
          const int c = (i >> 6) % NCH, s = i & 63, h = s >> 5;
          const int q = qbase + (i >> 6) / NCH * kFrag + (s & 31);
          v[u] = u32x4_t{0u, 0u, 0u, 0u};
          if (i0 + u < PER && i < NV && q < A.b) {
            if constexpr (CT == MIPS_BF16) {
              if (A.qraw_f32) {
                const float* p = (const float*)A.qraw + (int64_t)q * D + 16 * c + 8 * h;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  v[u][t] = (uint32_t)f32_to_bf16(p[2 * t]) | ((uint32_t)f32_to_bf16(p[2 * t + 1]) << 16);
              } else {
                const uint32_t* p = (const uint32_t*)((const uint16_t*)A.qraw + (int64_t)q * D + 16 * c + 8 * h);
#pragma unroll
                for (int t = 0; t < 4; ++t) v[u][t] = p[t];
              }
            } else {
              const float* p = (const float*)A.qraw + (int64_t)q * D + 8 * c + h;
#pragma unroll
              for (int t = 0; t < 4; ++t) v[u][t] = __float_as_uint(p[2 * t]);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kRawBatch; ++u) {
          const int i = (i0 + u) * kScoreThreads + threadIdx.x;
          if (i0 + u < PER && i < NV) {
            dst[i] = v[u];
            if (slice == 0 && i < n16) gdst[i] = v[u];
          }
        }
      }
      if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < A.nflags; i += kScoreThreads) A.ovf[i] = 0u;
        if (threadIdx.x < 2) A.nfail[threadIdx.x] = 0u;  // the rescue queue and rescan counts
      }
      for (int i = threadIdx.x; i < QB; i += kScoreThreads) {
        qid_lds[i] = qbase + i < A.b ? qbase + i : -1;
        seg_lds[i] = 0u;
      }
      if constexpr (NT > 0)
        for (int i = QB + threadIdx.x; i < QB * NT; i += kScoreThreads) seg_lds[i] = 0u;
    } else if (!rescue) {
      const int rows = min(QB, A.b32 - qbase);
      const u32x4_t* src = (const u32x4_t*)(A.qtile + (int64_t)qbase * D * E);
      u32x4_t* dst = (u32x4_t*)lds;
      const int n16 = rows * D * E / 16;
      for (int i0 = 0; i0 < PER; i0 += kFillBatch) {
        u32x4_t v[kFillBatch];
#pragma unroll
        for (int u = 0; u < kFillBatch; ++u) {
          const int i = (i0 + u) * kScoreThreads + threadIdx.x;
          v[u] = (i0 + u < PER && i < n16) ? src[i] : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kFillBatch; ++u) {
          const int i = (i0 + u) * kScoreThreads + threadIdx.x;
          if (i0 + u < PER && i < NV) dst[i] = v[u];
        }
      }
      for (int i = threadIdx.x; i < QB; i += kScoreThreads) {
        qid_lds[i] = qbase + i < A.b ? qbase + i : -1;
        seg_lds[i] = 0u;
      }
      if constexpr (NT > 0)
        for (int i = QB + threadIdx.x; i < QB * NT; i += kScoreThreads) seg_lds[i] = 0u;
    } else {
      for (int i = threadIdx.x; i < QB; i += kScoreThreads) {
        qid_lds[i] = qbase + i < nq_total ? (int)A.qlist[qbase + i] : -1;
        seg_lds[i] = 0u;
      }
      if constexpr (NT > 0)
        for (int i = QB + threadIdx.x; i < QB * NT; i += kScoreThreads) seg_lds[i] = 0u;
      __syncthreads();
      // gather the queued queries' operand rows: 16-byte slot s of chunk c of column
      // fragment qf comes from slot (q & 31) + 32 (s >> 5) of the same chunk of q's block
      u32x4_t* dst = (u32x4_t*)lds;
      for (int i0 = 0; i0 < PER; i0 += kFillBatch) {
        u32x4_t v[kFillBatch];
#pragma unroll
        for (int u = 0; u < kFillBatch; ++u) {
          const int i = (i0 + u) * kScoreThreads + threadIdx.x;
          v[u] = u32x4_t{0u, 0u, 0u, 0u};
          if (i0 + u < PER && i < NV) {
            const int s = i & 63, c = (i >> 6) % NCH, qf = (i >> 6) / NCH;
            const int qv = qid_lds[qf * kFrag + (s & 31)];
            const int q = (NT > 0 && qv >= 0) ? qv % A.b : qv;  // a masked pass queues (mask, query)
            if (q >= 0)
              v[u] = *(const u32x4_t*)(A.qtile + (int64_t)(q >> 5) * BLK + c * kChunkBytes +
                                       ((q & 31) + 32 * (s >> 5)) * 16);
          }
        }
#pragma unroll
        for (int u = 0; u < kFillBatch; ++u) {
          const int i = (i0 + u) * kScoreThreads + threadIdx.x;
          if (i0 + u < PER && i < NV) dst[i] = v[u];
        }
      }
    }
    __syncthreads();

    // Per query column: threshold and fp8 exponent, read from LDS once per query fragment
    // (registers are kept for the corpus stages and accumulators).
    for (int i = threadIdx.x; i < QB; i += kScoreThreads) {
      const int qg = qid_lds[i];
      float T = INFINITY;
      if constexpr (NT > 0) {
        // one threshold per mask (a rescued column scores its own mask only); the column's
        // own threshold, the lowest of them, gates the fast path
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float Tt = INFINITY;
          if (MODE == MODE_MAIN && qg >= 0 && t < A.nmask && (!rescue || qg / A.b == t)) {
            const uint32_t k = A.thr[rescue ? qg : t * A.b + qg];
            if (k != 0u) Tt = key_threshold(k);
          }
          thrt_lds[i * NT + t] = Tt;
          T = fminf(T, Tt);
        }
      } else if (MODE == MODE_MAIN && qg >= 0) {
        const uint32_t k = A.thr[qg];
        if (k != 0u) T = key_threshold(k);
      }
      thr_lds[i] = T;
      int e = CT == MIPS_INT8 ? __float_as_int(1.0f) : 127;
      if ((CT == MIPS_FP8_E4M3 || CT == MIPS_INT8) && qg >= 0)
        e = A.qexp[(NT > 0 && rescue) ? qg % A.b : qg];
      sexp_lds[i] = e;
    }
    __syncthreads();
    auto Tq = [&](int qf) __attribute__((always_inline)) { return thr_lds[qf * kFrag + (lane & 31)]; };
    auto sbq = [&](int qf) __attribute__((always_inline)) {
      return CT == MIPS_FP8_E4M3 ? sexp_lds[qf * kFrag + (lane & 31)] : 127;
    };
    // int8: a score is (int32 dot product * query scale) * row scale, each product rounded
    // to binary32, in the order of the quantised branch of `RecsysTwoTowerModel.forward`.
    auto qscale = [&](int qf) __attribute__((always_inline)) {
      return CT == MIPS_INT8 ? __int_as_float(sexp_lds[qf * kFrag + (lane & 31)]) : 1.0f;
    };
    auto qgq = [&](int qf) __attribute__((always_inline)) { return qid_lds[qf * kFrag + (lane & 31)]; };
    // list (query or virtual query) of query column c and mask t
    auto listid = [&](int c, int t) __attribute__((always_inline)) {
      const int qg = qid_lds[c];
      return (NT > 0 && !rescue) ? t * A.b + qg : qg;
    };

    int st_n = 0;  // staged survivors of this wave (wave-uniform; may exceed the capacity)

    // Appends the staged survivors to their queries' lists. Every workgroup owns one
    // segment of each query's list (segment = its corpus slice); positions come from LDS
    // counters, so no global atomic is needed. The counters also count what does not fit
    // the segment, which the final select sees as an overflow.
    auto flush = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int nst = min(st_n, kStageCap);
      constexpr int R = kStageCap / kWave;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int e = r * kWave + lane;
        if (e < nst) {
          const uint64_t ck = st_key[e];
          const int qc = st_q[e];
          const int64_t list = NT > 0 ? listid(qc / NTS, qc % NTS) : qid_lds[qc];
          if (rescue) {
            // a rescued list is one run for the whole pass: few lists and few survivors,
            // so one global atomic per survivor
            const uint32_t pos = atomicAdd(&A.rtail[list], 1u);
            if ((int64_t)pos < (int64_t)A.nseg * A.capw) A.cand[list * A.nseg * A.capw + pos] = ck;
          } else {
            const uint32_t pos = atomicAdd(&seg_lds[qc], 1u);
            if ((int64_t)pos < A.capw) A.cand[(list * A.nseg + slice) * A.capw + pos] = ck;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      st_n = 0;
    };

    // A stage's loads are unconditional: blocks past the end of the pass read the last
    // block again and are masked out, so the compiler's wait counts stay exact. Lane r < RM
    // (multi-mask: lane NT r + t, for mask t) also loads the exclusion word of block r.
    // Loaded values are kept as loaded until the stage is computed: a value derived from a
    // load in flight (the exclusion word with the padding rows set, the exponent of an fp8
    // row scale) is a use of that load, and the compiler would place it before the loop's
    // back edge with a wait for the load and so for every load issued before it, draining
    // the stages in flight once per iteration.
    auto word_block = [&](int64_t j0, bool& live) __attribute__((always_inline)) {
      const int rl = NT > 0 ? lane / NTS : lane;
      const int r = rl < RM ? rl : RM - 1;
      live = j0 + r < A.nfrag;
      const int64_t j = live ? j0 + r : A.nfrag - 1;
      return A.blk0 + ((MODE == MODE_SAMPLE) ? (int64_t)(((uint64_t)j * A.sample_step) >> 32) : j);
    };
    auto load_stage = [&](u32x4_t (&a)[RM][NCH], int (&sa)[RM], float (&sc)[RM][SCN], uint32_t& xraw,
                          int64_t j0) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        const int64_t j = min<int64_t>(j0 + r, A.nfrag - 1);
        const int64_t fr = A.blk0 + ((MODE == MODE_SAMPLE) ? (int64_t)(((uint64_t)j * A.sample_step) >> 32) : j);
        // one buffer descriptor per block (scalar base, range = the block's bytes) and a
        // 32-bit lane offset: no per-lane 64-bit addresses to keep live
        const __amdgpu_buffer_rsrc_t rs = block_rsrc(A.corpus + fr * BLK, (int)BLK);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          a[r][c] = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, c * kChunkBytes, 0));
        sa[r] = 127 << 23;  // the bits of a row scale of 1 (fp8: the row's own scale)
        if (CT == MIPS_FP8_E4M3) sa[r] = (int)__float_as_uint(A.row_scale[fr * kFrag + (lane & 31)]);
        if constexpr (CT == MIPS_INT8) {
          // rows 8q + 4 (lane >> 5) + (0..3) for q = 0..3: accumulator registers 4q..4q+3
          const __amdgpu_buffer_rsrc_t rsc = block_rsrc(A.row_scale + fr * kFrag, kFrag * 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4_t v = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsc, (lane >> 5) * 16, q * 32, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[r][4 * q + e] = __uint_as_float(v[e]);
          }
        }
      }
      // branch-free: without a bitmap, any readable word (masked to zero by stage_word); a
      // conditional load would make the compiler's wait counts conservative at the join
      bool live;
      const int64_t fr = word_block(j0, live);
      const uint32_t* wp;
      if constexpr (NT > 0) {
        const int mt = lane % NTS;
        wp = mt < A.nmask ? A.masks + (int64_t)mt * A.mask_words + fr : (const uint32_t*)A.corpus;
      } else {
        wp = A.exclude ? A.exclude + fr : (const uint32_t*)A.corpus;
      }
      xraw = *wp;
    };
    // The exclusion word of a stage's block (per lane, as loaded by load_stage) with the rows
    // past n, the rows before lo and every row of a block past the pass set; a mask past
    // the pass's count excludes every row.
    auto stage_word = [&](uint32_t xraw, int64_t j0) __attribute__((always_inline)) {
      bool live;
      const int64_t fr = word_block(j0, live);
      uint32_t keep, force = 0u;
      if constexpr (NT > 0) {
        const bool use = lane % NTS < A.nmask;
        keep = use ? ~0u : 0u;
        force = use ? 0u : ~0u;
      } else {
        keep = A.exclude ? ~0u : 0u;
      }
      uint32_t w = (xraw & keep) | force;
      const int64_t rows = A.n - fr * kFrag;
      if (rows < kFrag) w |= ~0u << rows;
      const int64_t below = A.lo - fr * kFrag;  // rows before the start of the id range
      if (below > 0) w |= below >= kFrag ? ~0u : (1u << below) - 1u;
      return live ? w : ~0u;
    };

    auto load_b = [&](u32x4_t (&bq)[NCH], int qf) __attribute__((always_inline)) {
      const u32x4_t* bsrc = (const u32x4_t*)(lds + (size_t)qf * BLK) + lane;
#pragma unroll
      for (int c = 0; c < NCH; ++c) bq[c] = bsrc[c * (kChunkBytes / 16)];
    };
    // MFMAs of one query fragment against the stage's RM blocks. With `next` >= 0 the
    // operand chunks are refilled from fragment `next` in LDS as soon as their last MFMA
    // has been issued, so the next fragment's operand streams in behind this one's.
    auto mfmas = [&](f32x16_t (&acc)[RM], const u32x4_t (&a)[RM][NCH], const int (&sa)[RM],
                     u32x4_t (&bq)[NCH], int sb, int next) __attribute__((always_inline)) {
      const u32x4_t* bsrc = (const u32x4_t*)(lds + (size_t)(next < 0 ? 0 : next) * BLK) + lane;
#pragma unroll
      for (int g = 0; g < RM; ++g) acc[g] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
        for (int g = 0; g < RM; ++g) mfma_step<CT>(acc[g], a[g], bq, sa[g], sb, s);
        if (next >= 0) {
          // chunks whose last use was step s: bf16 and int8 chunk s; fp8 chunks 2s, 2s+1;
          // f32 chunk s/4 after its fourth step
          if constexpr (CT == MIPS_BF16 || CT == MIPS_INT8) {
            bq[s] = bsrc[s * (kChunkBytes / 16)];
          } else if constexpr (CT == MIPS_FP8_E4M3) {
            bq[2 * s] = bsrc[2 * s * (kChunkBytes / 16)];
            bq[2 * s + 1] = bsrc[(2 * s + 1) * (kChunkBytes / 16)];
          } else {
            if ((s & 3) == 3) bq[s >> 2] = bsrc[(s >> 2) * (kChunkBytes / 16)];
          }
        }
      }
    };
    // A lane's 16 scores of block g: the accumulators, or for int8 the integer dot products
    // times the query scale sq, then times their rows' scales.
    auto vals = [&](const f32x16_t& acc, const float (&sc)[SCN], float sq, float (&x)[16]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (CT == MIPS_INT8)
          x[i] = ((float)__float_as_int(acc[i]) * sq) * sc[i];  // (a bit cast of a vector
                                                               // element lvalue would read
                                                               // element 0)
        else
          x[i] = acc[i];
      }
    };
    // Fast-path bound of a lane's best score in block g, one multiply per value. For int8 it
    // is max_i((a_i * s_i) * sq), the products in the other order: each order is within a
    // factor (1 + 2^-24)^2 of the exact a_i sq s_i, so a score of the filter's order that
    // reaches T implies this bound reaches gate(T) = T - |T| 2^-21.
    // The maximum of accumulators starts from kMaxSeed: the compiler then builds the chain
    // from v_max3 alone (raw MFMA results as the first operands of a plain v_max would each
    // take a quieting v_max first). The seed can only add false positives, which the slow
    // path resolves: max(seed, values) >= T exactly when some value is, unless T <= seed.
    constexpr float kMaxSeed = -4.0f;
    auto fastmax_into = [&](float x, const f32x16_t& acc, const float (&sc)[SCN]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        x = fmaxf(x, CT == MIPS_INT8 ? (float)__float_as_int(acc[i]) * sc[i] : acc[i]);
      return x;
    };
    auto fastmax = [&](const f32x16_t& acc, const float (&sc)[SCN], float sq) __attribute__((always_inline)) {
      if constexpr (CT == MIPS_INT8) {
        // products are canonical already: the chain starts from the first
        float x = (float)__float_as_int(acc[0]) * sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) x = fmaxf(x, (float)__float_as_int(acc[i]) * sc[i]);
        return x * sq;
      } else {
        return fastmax_into(kMaxSeed, acc, sc);
      }
    };
    auto gate = [&](float T) __attribute__((always_inline)) {
      return CT == MIPS_INT8 ? fmaf(-fabsf(T), 0x1p-21f, T) : T;  // (NaN for T = +inf: no pass)
    };

    // Main epilogue of one query fragment: one max per block (16 scores per lane) and one
    // ballot, branch-free so it interleaves with the next fragment's MFMAs. A block that
    // clears the threshold is resolved on the scalar unit (below).
    // Slow path of one block: per lane, a 16-bit mask of its values that pass: bit i <=>
    // y[i] >= T and its row (8 (i >> 2) + 4 (lane >> 5) + (i & 3)) is not set in the
    // block's word w (excluded or padding). The wave then walks the passing (lane, value)
    // pairs on the scalar unit, usually one, and stages each survivor for mask t.
    auto pass_walk = [&](const float (&y)[16], uint32_t w, float T, uint32_t idb, int qf,
                         int t) __attribute__((always_inline)) {
      uint32_t pm = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) pm |= (y[i] >= T ? 1u : 0u) << i;
      const uint32_t wl = w >> (4 * (lane >> 5));
      pm &= ~((wl & 0xFu) | ((wl >> 4) & 0xF0u) | ((wl >> 8) & 0xF00u) | ((wl >> 12) & 0xF000u));
      uint64_t H = __ballot(pm != 0u);
      while (H != 0ull) {
        const int L = __builtin_ctzll(H);
        H &= H - 1ull;
        uint32_t pl = (uint32_t)__builtin_amdgcn_readlane((int)pm, L);
        const int qcol = qf * kFrag + (L & 31);
        // column L's threshold key (T is per lane: each lane holds its own column's); the
        // walk compares keys, so that it stays on the scalar unit
        const uint32_t kTL = score_key(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(T), L)));
        while (pl != 0u) {
          const int i = __builtin_ctz(pl);
          pl &= pl - 1u;
          const uint32_t kv = score_key(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(y[i]), L)));
          const uint32_t id = idb + (uint32_t)(8 * (i >> 2) + 4 * (L >> 5) + (i & 3));
          // a rescue threshold is composite: at the threshold's own score only ids at or
          // below its id bound pass (rows tied with the k-th candidate cannot flood it)
          if (rescue && kv == kTL && id > A.thr_id[listid(qcol, t)]) continue;
          if (st_n < kStageCap) {
            if (lane == 0) {
              st_key[st_n] = composite(kv, id);
              st_q[st_n] = (uint16_t)(NT > 0 ? qcol * NTS + t : qcol);
            }
          } else if (lane == 0) {
            atomicOr(&A.ovf[listid(qcol, t)], 1u);  // no room: the list is rescued
          }
          ++st_n;
        }
      }
    };

    // (T and sq are the fragment's threshold and int8 query scale, read from LDS by the
    // caller; with two accumulator sets it reads them ahead of the next fragment's MFMAs,
    // since read after that fragment's operand reads were issued, their wait would wait
    // for those reads as well)
    auto epi_main = [&](const f32x16_t (&acc)[RM], const float (&sc)[RM][SCN], uint32_t xwv,
                        int64_t j0, int qf, float T, float sq) __attribute__((always_inline)) {
      const float Tg = gate(T);
      // one maximum over the stage's RM blocks and one compare (a single-mask pass); the
      // slow path takes each block's own maximum again
      bool any;
      float m[RM];
      if constexpr (NT == 0) {
        float x;
        if constexpr (CT == MIPS_INT8) {
          x = fastmax(acc[0], sc[0], 1.0f);
#pragma unroll
          for (int g = 1; g < RM; ++g) x = fastmax_into(x, acc[g], sc[g]);
          x = x * sq;
        } else {
          x = kMaxSeed;
#pragma unroll
          for (int g = 0; g < RM; ++g) x = fastmax_into(x, acc[g], sc[g]);
        }
        any = x >= Tg;
      } else {
        any = false;
#pragma unroll
        for (int g = 0; g < RM; ++g) {
          m[g] = fastmax(acc[g], sc[g], sq);
          any = any || (m[g] >= Tg);
        }
      }
      if (__builtin_expect(__ballot(any) != 0ull, 0)) {
#pragma unroll
        for (int g = 0; g < RM; ++g) {
          if constexpr (NT == 0) m[g] = fastmax(acc[g], sc[g], sq);
          if (__ballot(m[g] >= Tg) == 0ull) continue;
          const uint32_t idb = (uint32_t)((A.blk0 + j0 + g) * kFrag);
          float y[16];
          vals(acc[g], sc[g], sq, y);
          if constexpr (NT == 0) {
            pass_walk(y, (uint32_t)__builtin_amdgcn_readlane((int)xwv, g), T, idb, qf, 0);
          } else {
            // the block max reached the lowest of the column's thresholds; resolve only
            // the masks whose own threshold some lane's max reaches
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              if (t >= A.nmask) break;
              const float Tt = thrt_lds[(qf * kFrag + (lane & 31)) * NT + t];
              if (__ballot(m[g] >= gate(Tt)) == 0ull) continue;
              pass_walk(y, (uint32_t)__builtin_amdgcn_readlane((int)xwv, g * NT + t), Tt, idb, qf, t);
            }
          }
        }
      }
    };

    // Auxiliary epilogue. Dense pass: every score of the block goes to the query's list at
    // its id (0 for excluded and padding rows). Sample pass: the best eligible score of a
    // block is its delegate (key 0 if none is eligible); each half of the wave holds 16 of the
    // block's 32 rows, so the two lanes of a query's column combine their maxima. The stage's
    // RM delegates of a query form one slot, laid out del[tile / 16][query][tile % 16][RM],
    // so that each query's delegates lie in runs of 16 slots.
    auto epi_aux = [&](const f32x16_t (&acc)[RM], const float (&sc)[RM][SCN], uint32_t xwv,
                       int64_t j0, int qf) __attribute__((always_inline)) {
      const int qg = qgq(qf);
      const float sq = qscale(qf);
      if constexpr (MODE == MODE_DENSE) {
#pragma unroll
        for (int g = 0; g < RM; ++g) {
          const int64_t j = j0 + g;
          uint32_t wt[NTS];  // the block's word (per mask)
#pragma unroll
          for (int t = 0; t < NTS; ++t)
            wt[t] = (uint32_t)__builtin_amdgcn_readlane((int)xwv, NT > 0 ? g * NT + t : g);
          // The stores below are per lane (padding query columns are skipped). Their only
          // inputs are the accumulators, so without this pin the compiler may sink the
          // MFMAs, and the VALU work that feeds their per-lane scale operand, into the
          // lane-divergent branch, where inactive lanes leave the operand stale. The
          // volatile statement keeps the whole product in wave-uniform control flow.
          f32x16_t v = acc[g];
          asm volatile("" : "+v"(v));
          if (j < A.nfrag && qg >= 0) {
            float x[16];
            vals(v, sc[g], sq, x);
#pragma unroll
            for (int t = 0; t < NTS; ++t) {
              if (NT > 0 && t >= A.nmask) break;
              uint64_t* dst = A.cand + (int64_t)(NT > 0 ? t * A.b + qg : qg) * A.nseg * A.capw + j * kFrag;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int row = acc_row(i, lane);
                dst[row] = ((wt[t] >> row) & 1u)
                               ? 0ull
                               : composite(score_key(x[i]),
                                           (uint32_t)((A.blk0 + j) * kFrag + row));
              }
            }
          }
        }
      } else {
        const int qc = qbase + qf * kFrag + lane;
        const int64_t tt = j0 / RM;  // sample tile
#pragma unroll
        for (int t = 0; t < NTS; ++t) {
          if (NT > 0 && t >= A.nmask) break;
          uint32_t d[RM];
#pragma unroll
          for (int g = 0; g < RM; ++g) {
            const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)xwv, NT > 0 ? g * NT + t : g);
            float x[16];
            vals(acc[g], sc[g], sq, x);
            // The maximum starts from kMaxSeed, below every score of unit vectors; a block
            // whose maximum stays at or below it has no delegate (key 0). That can only
            // drop a delegate, so the bound stays proven.
            float mx = kMaxSeed;
            if (w == 0u) {
              // every row of the block is eligible (the usual case; w is wave-uniform): a
              // plain chain of v_max3
#pragma unroll
              for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[i]);
            } else {
              // Register i holds row acc_row(i, lane): bit 8 (i / 4) + i % 4 of w in lanes
              // 0-31, that bit + 4 in lanes 32-63. Its exclusion is thus a wave-uniform lane
              // mask, built on the scalar unit and applied by one select.
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int b0 = 8 * (i >> 2) + (i & 3);
                const uint64_t m = (((w >> b0) & 1u) ? 0x00000000FFFFFFFFull : 0ull) |
                                   (((w >> (b0 + 4)) & 1u) ? 0xFFFFFFFF00000000ull : 0ull);
                mx = fmaxf(mx, __builtin_amdgcn_inverse_ballot_w64(m) ? -INFINITY : x[i]);
              }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));  // the block's other 16 rows
            d[g] = (mx <= kMaxSeed) ? 0u : score_key(mx);
            asm volatile("" : "+v"(d[g]));  // computed in uniform control flow, as above
          }
          if constexpr (NT > 0) {
            // mask t's delegates are those of virtual query t * b + q
            if (lane < kFrag && qc < A.b) {
              uint32_t* dst = A.del + (((tt >> 4) * A.bv32 + t * A.b + qc) * 16 + (tt & 15)) * RM;
#pragma unroll
              for (int g = 0; g < RM; ++g) dst[g] = d[g];
            }
          } else if (lane < kFrag && qc < A.b32) {
            uint32_t* dst = A.del + (((tt >> 4) * A.b32 + qc) * 16 + (tt & 15)) * RM;
#pragma unroll
            for (int g = 0; g < RM; ++g) dst[g] = d[g];
          }
        }
      }
    };

    // One stage against every query fragment, software-pipelined: the MFMAs of fragment
    // qf+1 are issued before the epilogue of fragment qf, so the epilogue (and its rare
    // path) runs while the matrix pipe works on the next fragment.
    auto compute_stage = [&](const u32x4_t (&a)[RM][NCH], const int (&sa_raw)[RM],
                             const float (&sc)[RM][SCN], uint32_t xraw,
                             int64_t j0) __attribute__((always_inline)) {
      const uint32_t xwv = stage_word(xraw, j0);
      int sa[RM];  // the MFMA's block scale operand: the biased exponent of the row scale
#pragma unroll
      for (int g = 0; g < RM; ++g) sa[g] = (int)(((uint32_t)sa_raw[g] >> 23) & 0xFFu);
      if constexpr (SINGLE) {
        // one accumulator set: fragment qf's MFMAs, then its epilogue (the other wave on
        // the SIMD keeps the matrix pipe busy meanwhile); the operand of fragment qf+1
        // streams in from LDS behind the MFMAs
        f32x16_t acc1[RM];
        u32x4_t bq1[NCH];
        load_b(bq1, 0);
        static_for<NQF>([&](auto qfc) __attribute__((always_inline)) {
          constexpr int qf = decltype(qfc)::value;
          // issue priority while this wave issues its MFMAs, none during its epilogue: the
          // two waves of a SIMD then take turns on the matrix pipe instead of sharing it and
          // reaching their epilogues together
          // the fragment's threshold is read ahead of the operand refills issued among its
          // MFMAs, so that the compare waits for that read alone, not for the refills too
          const float Tf = Tq(qf);
          __builtin_amdgcn_s_setprio(3);
          mfmas(acc1, a, sa, bq1, sbq(qf), qf + 1 < NQF ? qf + 1 : -1);
          __builtin_amdgcn_s_setprio(0);
          epi_main(acc1, sc, xwv, j0, qf, Tf, qscale(qf));
        });
        return;
      }
      f32x16_t acc[2][RM];
      u32x4_t bq[NCH];
      load_b(bq, 0);
      mfmas(acc[0], a, sa, bq, sbq(0), NQF > 1 ? 1 : -1);
      static_for<NQF>([&](auto qfc) __attribute__((always_inline)) {
        constexpr int qf = decltype(qfc)::value;
        constexpr int cur = qf & 1;
        float T = 0.0f, sq = 1.0f;
        if constexpr (MODE == MODE_MAIN) {
          T = Tq(qf);
          sq = qscale(qf);
        }
        if constexpr (qf + 1 < NQF) {
          if constexpr (MODE == MODE_MAIN) __builtin_amdgcn_s_setprio(3);  // as above
          mfmas(acc[cur ^ 1], a, sa, bq, sbq(qf + 1), qf + 2 < NQF ? qf + 2 : -1);
          if constexpr (MODE == MODE_MAIN) __builtin_amdgcn_s_setprio(0);
        }
        if constexpr (MODE == MODE_MAIN) {
          epi_main(acc[cur], sc, xwv, j0, qf, T, sq);
        } else {
          epi_aux(acc[cur], sc, xwv, j0, qf);
          // the auxiliary epilogues have no branch that would bound the scheduler's region;
          // without this fence it interleaves whole stages and runs out of registers
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    };

    // NS-stage software pipeline over this wave's stage tiles (a stage every kScoreWaves
    // tiles): while stage i is multiplied against every query, stages i+1 .. i+NS-1 are in
    // flight. The bytes in flight per SIMD set the HBM bandwidth (Little's law at several
    // microseconds of loaded latency), hence NS - 1 = 2 stages of 16 KiB per SIMD. The
    // sample and dense passes hold one stage less with two waves per SIMD: their epilogues
    // need the registers, and they run few stages per wave.
    constexpr int NS = (SINGLE || (MODE != MODE_MAIN && score_wps(CT, D) == 2)) ? 2 : kPipeStages;
    u32x4_t a[NS][RM][NCH];
    int sa[NS][RM];
    float sc[NS][RM][SCN];
    uint32_t xw[NS];
    int64_t t = t_begin + wave;
    auto tile = [&](int64_t tt) __attribute__((always_inline)) { return tt < t_end ? tt * RM : A.nfrag; };
    if (t < t_end) {
      static_for<NS - 1>([&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        load_stage(a[u], sa[u], sc[u], xw[u], tile(t + u * kScoreWaves));
      });
      // one pipeline step; returns true after the wave's last stage. The steps are chained
      // with || so that the exits are plain branches and every wait count stays exact.
      auto step = [&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        constexpr int ld = (u + NS - 1) % NS;
        load_stage(a[ld], sa[ld], sc[ld], xw[ld], tile(t + (u + NS - 1) * kScoreWaves));
        if (MODE == MODE_MAIN && st_n > kStageCap - kStageBurst) flush();
        compute_stage(a[u], sa[u], sc[u], xw[u], (t + u * kScoreWaves) * RM);
        return t + (u + 1) * kScoreWaves >= t_end;
      };
      static_assert(NS == 2 || NS == 3, "the step chains below are written for two or three stages");
      if constexpr (NS == 3) {
        while (!(step(std::integral_constant<int, 0>{}) || step(std::integral_constant<int, 1>{}) ||
                 step(std::integral_constant<int, 2>{})))
          t += NS * kScoreWaves;
      } else {
        while (!(step(std::integral_constant<int, 0>{}) || step(std::integral_constant<int, 1>{})))
          t += NS * kScoreWaves;
      }
    }
    if (MODE == MODE_MAIN) {
      if (st_n > 0) flush();
      // this workgroup's segment counts of the block's queries (a rescued list counts
      // through its tail instead)
      __syncthreads();
      for (int i = threadIdx.x; i < QB * NTS && !rescue; i += kScoreThreads) {
        const int c = i / NTS, t = i % NTS;
        const int q = qid_lds[c];
        if (q >= 0 && (NT == 0 || (t < A.nmask && (!rescue || q / A.b == t))))
          A.segcnt[(int64_t)listid(c, t) * A.nseg + slice] = seg_lds[i];
      }
    }
  }
}

template <int CT, int D, int NQF, int MODE, int NT>
static int launch_score(const ScoreArgs& A, int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr int lds = score_lds_bytes(CT, D, NQF, NT);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)score_kernel<CT, D, NQF, MODE, NT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  if (e0 && e1)
    // timing events taken by the dispatch itself (events recorded as packets of their
    // own around the launch would add a dispatch gap on each side)
    hipExtLaunchKernelGGL((score_kernel<CT, D, NQF, MODE, NT>), dim3(grid), dim3(score_threads(CT, D)), lds, s,
                          e0, e1, 0, A);
  else
    hipLaunchKernelGGL((score_kernel<CT, D, NQF, MODE, NT>), dim3(grid), dim3(score_threads(CT, D)), lds, s, A);
  return check_launch();
}

template <int CT, int D, int MODE, int NT>
int launch_score_nqf(int nqf, const ScoreArgs& A, int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (nqf) {
    case 1: return launch_score<CT, D, 1, MODE, NT>(A, grid, s, e0, e1);
    case 2: return launch_score<CT, D, 2, MODE, NT>(A, grid, s, e0, e1);
    case 4:
      if constexpr (nqf_fits(CT, D, 4, NT)) return launch_score<CT, D, 4, MODE, NT>(A, grid, s, e0, e1);
      break;
    case 8:
      if constexpr (NT == 0 && nqf_fits(CT, D, 8)) return launch_score<CT, D, 8, MODE, NT>(A, grid, s, e0, e1);
      break;
    case 16:
      if constexpr (NT == 0 && nqf_fits(CT, D, 16)) return launch_score<CT, D, 16, MODE, NT>(A, grid, s, e0, e1);
      break;
  }
  return MIPS_ERR_UNSUPPORTED;
}

}  // namespace mips
