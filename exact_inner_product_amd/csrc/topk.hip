// topk.hip -- exhaustive inner-product top-K for gfx950 (MI355X).
//
// The serving step of two-tower retrieval: score a batch of normalised user vectors
// against the whole normalised index by dot product and keep each user's K best
// (`RecsysTwoTowerModel.forward` in recsys_two_tower_model.py; Phoenix README, "How
// Retrieval Works", step 4). The score matrix is never written out. One call runs:
//
//   prep_queries     queries -> MFMA operand layout (E4M3 + power-of-two scale for an
//                    fp8 corpus); clears the per-query flags.
//   score<SAMPLE>    sample pass: scores a strided sample of G 32-row blocks and writes,
//                    per (block, query), the best eligible score of the block ("delegate").
//   sample_threshold per query: the K-th largest delegate is a proven lower bound of the
//                    K-th best score (K distinct blocks hold an item at least that good);
//                    a higher delegate rank, scaled to the sample fraction, gives an
//                    estimated threshold that about 2-3 K items of the whole corpus clear.
//   score<MAIN>      streams the packed corpus HBM -> VGPR (1 KiB coalesced wave loads)
//                    against the query block staged in LDS on the 32x32 MFMA; keeps in
//                    registers only a per-lane max; blocks whose max clears the query's
//                    threshold are resolved item by item (exclusion bitmap, threshold) and
//                    the survivors are appended to the query's candidate list.
//   final_select     per query, a radix select over 64-bit composite keys (score key << 32 |
//                    ~id) of its candidates and a rank sort: score descending, then id
//                    ascending. A query whose estimated threshold proved too high (fewer
//                    than K candidates) or whose list overflowed is queued for a rescue pass
//                    with a proven threshold, and then selected again.
//   score<MAIN>      rescue pass over the queued queries only (exits at once if none).
//   final_select     second round for the rescued queries; anything still unresolved is
//                    rescanned exactly by its workgroup.
//
// Corpora too small for a useful sample (fewer blocks than about 2K) take a dense pass
// instead: every score is written to the query's list, indexed by id, and selected.
#include <algorithm>
#include <cmath>

#include "common.h"
#include "host.h"
#include "score_api.h"
#include "select.h"

namespace mips {


// ------------------------------------------------------------------ query prep
// Queries -> MFMA operand tile (the packed layout of the corpus, 32 queries per block).
// One workgroup of 64 threads per (32-query block, 1 KiB chunk); thread s writes slot s.
// The wave first copies the block's 32 query rows into LDS with coalesced 4-byte loads,
// all in flight at once; every value it needs, and each row's max |q|, then come from LDS.
// For an fp8 or int8 corpus each query row is quantised with its own scale (the corpus
// rule): lanes s and s + 32 each take the max over half the row's dimensions and combine
// them. Clears the per-query flags.
template <int CT, int QT, int D>
__global__ __launch_bounds__(64) void prep_queries_kernel(const void* __restrict__ queries, int b,
                                                          uint8_t* __restrict__ qtile,
                                                          int* __restrict__ qexp,
                                                          uint32_t* __restrict__ ovf, int nflags,
                                                          uint32_t* __restrict__ nfail) {
  constexpr int NCH = chunks_per_block(CT, D);
  constexpr int RW = D * (QT == MIPS_F32 ? 4 : 2) / 4;  // 4-byte words per query row
  constexpr int RWP = RW + 1;  // LDS row stride: odd, so the 32 rows of a column lie in 32 banks
  __shared__ uint32_t rows[kFrag * RWP];
  const int lane = threadIdx.x;
  const int qb = blockIdx.x / NCH, c = blockIdx.x % NCH;
  const int q = qb * kFrag + (lane & 31);
  const int nrows = min(kFrag, b - qb * kFrag);
  const uint32_t* src = (const uint32_t*)queries + (int64_t)qb * kFrag * RW;
  // Unconditional loads (words past the batch read its last word and are stored as zero): a
  // load under a branch would be waited for before the next one is issued.
  const int nw = nrows * RW;
  static_assert(kFrag * RW % 64 == 0, "whole rounds of the 64 lanes");
#pragma unroll 32
  for (int it = 0; it < kFrag * RW / 64; ++it) {
    const int i = it * 64 + lane;
    const uint32_t x = src[min(i, nw - 1)];
    rows[(i / RW) * RWP + i % RW] = i < nw ? x : 0u;
  }
  __syncthreads();
  auto val = [&](int dim) -> float {
    const uint32_t* r = rows + (lane & 31) * RWP;
    if (QT == MIPS_F32) return __uint_as_float(r[dim]);
    return bf16_to_f32((uint16_t)(r[dim >> 1] >> (16 * (dim & 1))));
  };
  float sinv = 1.0f, sq = 1.0f;
  float m = 0.0f;  // max |q| of this lane's row (fp8 and int8): half each, then combined
  if (CT == MIPS_FP8_E4M3 || CT == MIPS_INT8) {
    const int h = lane >> 5;
#pragma unroll 8
    for (int j = h * (D / 2); j < (h + 1) * (D / 2); ++j) m = fmaxf(m, fabsf(val(j)));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
  }
  if (CT == MIPS_FP8_E4M3) {
    int t = e4m3_scale_exp(m);
    t = t < -126 ? -126 : (t > 127 ? 127 : t);
    sinv = exp2_int(-t);
    if (c == 0 && lane < 32) qexp[q] = t + 127;
  } else if (CT == MIPS_INT8) {
    sq = i8_scale(m);
    if (c == 0 && lane < 32) qexp[q] = __float_as_int(sq);
  }
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (CT == MIPS_F32) {
    for (int t = 0; t < 4; ++t) v[t] = __float_as_uint(val(slot_dim(CT, c, lane, t)));
  } else if (CT == MIPS_BF16) {
    for (int t = 0; t < 8; t += 2)
      v[t >> 1] = (uint32_t)f32_to_bf16(val(slot_dim(CT, c, lane, t))) |
                  ((uint32_t)f32_to_bf16(val(slot_dim(CT, c, lane, t + 1))) << 16);
  } else if (CT == MIPS_INT8) {
    for (int t = 0; t < 16; ++t)
      v[t >> 2] |= f32_to_i8(val(slot_dim(CT, c, lane, t)) / sq) << (8 * (t & 3));
  } else {
    for (int t = 0; t < 16; ++t)
      v[t >> 2] |= (uint32_t)f32_to_e4m3(val(slot_dim(CT, c, lane, t)) * sinv) << (8 * (t & 3));
  }
  *(u32x4_t*)(qtile + (int64_t)qb * block_bytes(CT, D) + (int64_t)c * kChunkBytes + lane * 16) = v;
  // the overflow flag of every list (query, or virtual query of a multi-mask pass)
  for (int i = blockIdx.x * 64 + lane; i < nflags; i += gridDim.x * 64) ovf[i] = 0u;
  if (blockIdx.x == 0 && lane < 2) nfail[lane] = 0u;  // the rescue queue and rescan counts
}

// ------------------------------------------------------------ sampled threshold
// Per query, from the G delegates (best eligible score per sampled block of 32 rows):
// tb, a proven lower bound of the K-th best score (at least K delegates, i.e. K distinct
// blocks, reach it), and te >= tb at delegate rank r (r <= K), the estimate the main pass
// filters with.
// Both come from one histogram of the delegate scores over kThrBins equal bins of
// [-kThrRange, kThrRange] (scores outside fall into the end bins) and a suffix scan: the
// threshold of rank r is the lower edge of the bin holding the r-th largest delegate, less
// a margin that absorbs the rounding of the bin computation, so at least r delegates
// reach it. Key 0 means "no bound" (fewer than K, resp. r, eligible sampled blocks).
constexpr int kThrBins = 4096;
constexpr float kThrRange = 1.25f;  // > (1 + 2^-4)^2, the largest fp8 score of unit vectors

__device__ __forceinline__ int thr_bin(float s) {
  const float x = (s + kThrRange) * ((float)kThrBins / (2.0f * kThrRange));
  const int b = (int)floorf(x);
  return b < 0 ? 0 : (b >= kThrBins ? kThrBins - 1 : b);
}
__device__ __forceinline__ uint32_t thr_bin_key(int b) {
  if (b <= 0) return 0u;  // the lowest bin is open below: no bound
  const float e = -kThrRange + (float)b * (2.0f * kThrRange / (float)kThrBins);
  return score_key(e - 1e-5f);
}

__global__ __launch_bounds__(kSelThreads) void sample_threshold_kernel(const uint32_t* __restrict__ del,
                                                                       int ntiles, int slot, int b32, int b,
                                                                       int k, int r, uint32_t* __restrict__ thr,
                                                                       uint32_t* __restrict__ thrb) {
  constexpr int PER = kThrBins / kSelThreads;  // bins per thread
  __shared__ uint32_t hist[kThrBins];
  __shared__ uint32_t wsum[kSelThreads / kWave];
  __shared__ int found[2];
  const int q = blockIdx.x;
  if (q >= b) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int i = t; i < kThrBins; i += kSelThreads) hist[i] = 0u;
  if (t < 2) found[t] = 0;
  __syncthreads();
  // the query's delegates: runs of 16 slots of `slot` delegates each (one slot per sample
  // tile), 4 * slot 16-byte vectors per run; consecutive threads read consecutive vectors,
  // eight loads in flight per thread before any histogram update
  const int ngroups = (ntiles + 15) / 16;
  const int nvec = 4 * slot;  // slot is 1, 2 or 4
  const int total = ngroups * nvec;
  for (int j0 = 0; j0 < total; j0 += kSelThreads * 8) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * kSelThreads + t;
      v[u] = u32x4_t{0u, 0u, 0u, 0u};
      if (j < total)
        v[u] = *((const u32x4_t*)(del + ((int64_t)(j / nvec) * b32 + q) * 16 * slot) + j % nvec);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * kSelThreads + t;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // slots of tiles past the end of the pass are never written
        const int tile = (j / nvec) * 16 + ((j % nvec) * 4 + e) / slot;
        if (j < total && tile < ntiles && v[u][e] != 0u)
          atomicAdd(&hist[thr_bin(key_score(v[u][e]))], 1u);
      }
    }
  }
  __syncthreads();
  // thread t owns bins [t*PER, (t+1)*PER); the suffix sum over threads above t gives the
  // count of delegates in higher bins
  uint32_t own = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) own += hist[t * PER + i];
  // inclusive suffix scan over the wave (lanes above), then over waves
  uint32_t c = own;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_down(c, o, kWave);
    if (lane + o < kWave) c += u;
  }
  if (lane == 0) wsum[w] = c;
  __syncthreads();
  for (int i = w + 1; i < kSelThreads / kWave; ++i) c += wsum[i];
  uint32_t above = c - own;  // delegates in bins above this thread's range
  // walk this thread's bins from the top; record the bins where ranks r and k are reached
  // (found[] holds bin + 1; exactly one thread reaches each rank)
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) {
    const uint32_t h = hist[t * PER + i];
    if (above < (uint32_t)r && above + h >= (uint32_t)r) found[0] = t * PER + i + 1;
    if (above < (uint32_t)k && above + h >= (uint32_t)k) found[1] = t * PER + i + 1;
    above += h;
  }
  __syncthreads();
  if (t == 0) {
    const uint32_t tb = found[1] > 0 ? thr_bin_key(found[1] - 1) : 0u;
    const uint32_t te = found[0] > 0 ? thr_bin_key(found[0] - 1) : 0u;
    thr[q] = te > tb ? te : tb;
    thrb[q] = tb;
  }
}

// ---------------------------------------------------------------- final select
struct SelectArgs {
  const uint8_t* corpus;
  const float* row_scale;
  const uint32_t* exclude;
  int64_t excl_rw;      // 0: one bitmap for every query; > 0: query q's row at q * excl_rw
  const uint32_t* masks;  // multi-mask pass: list q is mask q / breal of query q % breal
  int64_t mask_words;
  int breal;              // 0: one result set, list q is query q
  const uint8_t* qtile;
  const int* qexp;
  int64_t n;            // rows [lo, n) take part
  int64_t lo;
  int b;
  int k;
  int64_t capw;         // entries per list segment
  int nseg;             // segments per query list
  int nseg_used;        // segments written by the pass being selected from
  int cache_n;          // entries of the LDS candidate cache (sel_cache_entries(k))
  int64_t dense_count;  // > 0: lists hold one slot per row (0 = empty), this many
  uint32_t* thr;
  uint32_t* thrb;
  uint32_t* thr_id;     // id bound of a rescue's composite threshold
  uint32_t* rtail;      // survivors of a rescued list (its contiguous run's tail)
  const uint32_t* segcnt;
  uint32_t* ovf;
  const uint64_t* cand;
  uint32_t* nfail;      // [0]: lists queued for rescue; [1]: lists resolved by the rescan
  uint32_t* flist;
  float* out_scores;
  int32_t* out_ids;
};

// Writes query q's sorted keys (descending) and pads the rest with (-inf, -1).
__device__ void write_out(const SelectArgs& A, int q, const uint64_t* s, int cnt) {
  for (int t = threadIdx.x; t < A.k; t += kSelThreads) {
    float sc = -INFINITY;
    int32_t id = -1;
    if (t < cnt && s[t] != 0ull) {
      sc = key_score((uint32_t)(s[t] >> 32));
      id = (int32_t)composite_id(s[t]);
    }
    A.out_scores[(int64_t)q * A.k + t] = sc;
    A.out_ids[(int64_t)q * A.k + t] = id;
  }
}

// Exact rescan of query q: VALU dot products in dimension order, candidates buffered in
// LDS behind a composite-key threshold that rises whenever the buffer is compacted to
// its k best.
template <int CT, int D>
__device__ void fallback_scan(const SelectArgs& A, int q, uint64_t thr, uint64_t* buf,
                              uint64_t* sel_buf, SelScratch& S, float* qv, uint32_t* nbuf_p) {
  // list q: query qr, rows excluded by the bitmap row xq (or the mask of a multi-mask pass)
  const int qr = A.breal > 0 ? q % A.breal : q;
  const uint32_t* xq = A.breal > 0 ? A.masks + (int64_t)(q / A.breal) * A.mask_words
                                   : (A.exclude ? A.exclude + (int64_t)q * A.excl_rw : nullptr);
  for (int j = threadIdx.x; j < D; j += kSelThreads) {
    const int64_t off = (int64_t)(qr >> 5) * block_bytes(CT, D) + packed_offset(CT, D, qr & 31, j);
    float v;
    if (CT == MIPS_F32)
      v = *(const float*)(A.qtile + off);
    else if (CT == MIPS_BF16)
      v = bf16_to_f32(*(const uint16_t*)(A.qtile + off));
    else if (CT == MIPS_INT8)
      v = (float)(int8_t)A.qtile[off];  // the query scale is applied to the sum
    else
      v = e4m3_to_f32(A.qtile[off]) * exp2_int(A.qexp[qr] - 127);
    qv[j] = v;
  }
  if (threadIdx.x == 0) *nbuf_p = 0u;
  __syncthreads();
  constexpr int kRound = kSelThreads * 4;
  for (int64_t base = A.lo; base < A.n; base += kRound) {
    if (*nbuf_p + (uint32_t)kRound > (uint32_t)A.cache_n) {
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
      if (i >= A.n || (xq && ((xq[i >> 5] >> (i & 31)) & 1u))) continue;
      float s = 0.0f;
      for (int j = 0; j < D; ++j) {
        const int64_t off = packed_offset(CT, D, i, j);
        float c;
        if (CT == MIPS_F32)
          c = *(const float*)(A.corpus + off);
        else if (CT == MIPS_BF16)
          c = bf16_to_f32(*(const uint16_t*)(A.corpus + off));
        else if (CT == MIPS_INT8)
          c = (float)(int8_t)A.corpus[off];
        else
          c = e4m3_to_f32(A.corpus[off]);
        s = fmaf(qv[j], c, s);
      }
      if (CT == MIPS_FP8_E4M3) s *= A.row_scale[i];
      // int8: the sum of code products is an integer below 2^24, exact in fp32 as in the
      // MFMA path; then the query scale and the row scale, in the score pass's order
      if (CT == MIPS_INT8) s = (s * __int_as_float(A.qexp[qr])) * A.row_scale[i];
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

// Exclusive prefix sum over the workgroup's threads; returns (exclusive, total).
__device__ inline uint2 block_exclusive_sum(uint32_t v, uint32_t* wsum) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t c = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_up(c, o, kWave);
    if (lane >= o) c += u;
  }
  if (lane == kWave - 1) wsum[w] = c;
  __syncthreads();
  uint32_t before = 0u, total = 0u;
  for (int i = 0; i < kSelThreads / kWave; ++i) {
    if (i < w) before += wsum[i];
    total += wsum[i];
  }
  __syncthreads();
  return make_uint2(before + c - v, total);
}

// Queues list q for the rescue pass with the composite threshold (key nt, id bound nid);
// `every` also sets the proven bound to the every-row key. One thread per list.
__device__ inline void queue_rescue(const SelectArgs& A, int q, uint32_t nt, uint32_t nid,
                                    bool every) {
  const uint32_t slot = atomicAdd(A.nfail, 1u);
  A.flist[slot] = (uint32_t)q;
  A.thr[q] = nt;
  A.thr_id[q] = nid;
  if (every) A.thrb[q] = nt;
  A.ovf[q] = 0u;
  A.rtail[q] = 0u;
}

// The exact rescan of list q (the last resort), counted in nfail[1].
template <int CT, int D>
__device__ void rescan(const SelectArgs& A, int q, uint64_t* cache, uint64_t* sel_buf,
                       SelScratch& S, float* qv, uint32_t* nbuf) {
  if (threadIdx.x == 0) atomicAdd(A.nfail + 1, 1u);
  fallback_scan<CT, D>(A, q, 0ull, cache, sel_buf, S, qv, nbuf);
}

// Lists of at most this many candidates (and at most 4 k) are sorted whole instead of
// radix-selected first; for a k much smaller than the list, selecting first is cheaper.
constexpr int kSortAll = 512;

// Threshold key of -infinity: a pass with it keeps every eligible row.
constexpr uint32_t kEveryRowKey = 0x007FFFFFu;

// One workgroup per query. Round 0 covers the batch; round 1 the queries queued by round 0.
// A query's candidates lie in segments (one per workgroup of the pass that found them);
// thread s handles segment s.
template <int CT, int D>
__global__ __launch_bounds__(kSelThreads) void final_select_kernel(SelectArgs A, int round) {
  extern __shared__ __attribute__((aligned(16))) uint64_t cache[];  // A.cache_n entries
  __shared__ uint64_t sel_buf[MIPS_K_MAX];
  __shared__ SelScratch S;
  __shared__ float qv[D];
  __shared__ uint32_t nbuf;
  __shared__ uint32_t wsum[kSelThreads / kWave];
  int q = blockIdx.x;
  if (round > 0) {
    if ((uint32_t)q >= *A.nfail) return;
    q = (int)A.flist[q];
  }
  if (q >= A.b) return;
  const int t = threadIdx.x;
  const uint64_t* qlist = A.cand + (int64_t)q * A.nseg * A.capw;
  // One bitmap per query: the score passes apply none, so the query's own row filters its
  // candidates here (an excluded candidate reads as key 0, below every real key).
  const bool own = A.excl_rw > 0;
  const uint32_t* xrow = own ? A.exclude + (int64_t)q * A.excl_rw : nullptr;
  auto excluded = [&](uint64_t key) {
    const uint32_t id = composite_id(key);
    return ((xrow[id >> 5] >> (id & 31)) & 1u) != 0u;
  };
  int64_t c;
  bool cached;
  if (A.dense_count > 0) {
    // dense list: one slot per row; empty slots (key 0) are not candidates, so select
    // among the others only and no tie at the boundary involves an empty slot
    c = A.dense_count;
    cached = c <= A.cache_n;
    if (t == 0) nbuf = 0u;
    __syncthreads();
    uint32_t mine = 0u;
    for (int64_t i = t; i < c; i += kSelThreads) {
      uint64_t key = qlist[i];
      if (own && key != 0ull && excluded(key)) key = 0ull;
      if (cached) cache[i] = key;
      mine += key != 0ull;
    }
    atomicAdd(&nbuf, mine);
    __syncthreads();
    const int r = (int)min<int64_t>((int64_t)nbuf, A.k);
    if (cached && c <= kSortAll && c <= 4 * (int64_t)A.k) {
      // few slots: one sort of all of them (empty slots, key 0, sink to the end)
      bitonic_sort_desc(cache, (int)c);
      write_out(A, q, cache, r);
      return;
    }
    if (r > 0) {
      Sel64 sel{0ull, 0ull};
      if (cached) {
        auto get = [&](int64_t i) { return cache[i]; };
        if (c > r) sel = select_top(get, c, r, S);
        gather_sort(get, c, r, sel, sel_buf, &S.hist[0]);
      } else {
        auto get = [&](int64_t i) {
          const uint64_t key = qlist[i];
          return own && key != 0ull && excluded(key) ? 0ull : key;
        };
        if (c > r) sel = select_top(get, c, r, S);
        gather_sort(get, c, r, sel, sel_buf, &S.hist[0]);
      }
    }
    write_out(A, q, sel_buf, r);
    return;
  }
  // The list's words, issued together: its thresholds, overflow flag, rescued-run tail and
  // segment counts (each thread reads a segment count in bounds; only those of the segments
  // the pass wrote are used).
  uint32_t tu = A.thr[q], tb = A.thrb[q];
  uint32_t ovq = A.ovf[q];
  const uint32_t rt_raw = A.rtail[q];
  const uint32_t cnt_t = A.segcnt[(int64_t)q * A.nseg + min(t, A.nseg_used - 1)];
  // (passed through one empty asm statement, so that the compiler issues every load before
  // the first use of any of them instead of waiting for each in turn)
  asm volatile("" : "+v"(tu), "+v"(tb), "+v"(ovq) : "v"(cnt_t), "v"(rt_raw));
  const uint32_t rtq = round == 0 ? 0u : rt_raw;
  if (tu == 0u) {
    // No sampled bound (fewer than K sampled blocks hold an eligible row, so the query has
    // few eligible rows): the rescue pass gathers every eligible row on the MFMA path, and
    // its list is complete unless it overflows.
    if (round > 0) {
      rescan<CT, D>(A, q, cache, sel_buf, S, qv, &nbuf);
      return;
    }
    if (t == 0) queue_rescue(A, q, kEveryRowKey, 0xFFFFFFFFu, true);
    return;
  }
  // segment s: found (counted by the pass) and stored (what fits the segment). A rescued
  // list (round 1) is one run of nseg * capw entries with its count in rtail; it is read
  // as nseg segments of capw.
  uint32_t found, mine;
  int64_t total;  // everything the pass found for this list
  if (round == 0) {
    found = t < A.nseg_used ? cnt_t : 0u;
    mine = found < (uint32_t)A.capw ? found : (uint32_t)A.capw;
  } else {
    const int64_t r = (int64_t)rtq - (int64_t)t * A.capw;
    found = 0u;
    mine = t < A.nseg && r > 0 ? (uint32_t)min<int64_t>(r, A.capw) : 0u;
  }
  const uint2 so = block_exclusive_sum(mine, wsum);
  const uint2 sf = block_exclusive_sum(found, wsum);
  const int64_t stored = so.y;
  total = round == 0 ? (int64_t)sf.y : (int64_t)rtq;
  c = total;
  // Visits the thread's stored entries (its segment), 8 per round trip: unconditional loads
  // of stored entries (the last one again past the end), so that all 8 are in flight at
  // once. An entry the query's own bitmap excludes reads as key 0, below every real key.
  const uint64_t* seg = qlist + (int64_t)t * A.capw;
  auto each = [&](auto f) {
    for (uint32_t i0 = 0; i0 < mine; i0 += 8) {
      uint64_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = seg[min(i0 + e, mine - 1)];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (i0 + e < mine) f(own && excluded(v[e]) ? 0ull : v[e]);
    }
  };
  // eligible: the stored candidates the query's own bitmap keeps (all without one)
  int64_t eligible = stored;
  if (own) {
    if (t == 0) nbuf = 0u;
    __syncthreads();
    uint32_t keep = 0u;
    each([&](uint64_t key) { keep += key != 0ull; });
    atomicAdd(&nbuf, keep);
    __syncthreads();
    eligible = nbuf;
  }
  __syncthreads();
  const bool over = stored < c || ovq != 0u;
  // Fewer than k candidates: final when the threshold was the proven bound. With one
  // bitmap per query the sample pass applied none, so its bound is not proven and a short
  // list is always rescued; at the bound itself only the exact rescan is left.
  const bool shortfall = !over && tu != kEveryRowKey && eligible < A.k && (tu > tb || own);
  if (over || shortfall) {
    if (round > 0 || (shortfall && tu == tb)) {
      rescan<CT, D>(A, q, cache, sel_buf, S, qv, &nbuf);
      return;
    }
    // Rescue threshold: the proven bound after a shortfall (every row if the sample proved
    // none); after an overflow, the composite key of the k-th best stored candidate (k real
    // items reach it): rows above its score, and rows at its score with an id at or below
    // its id, so rows tied with it cannot overflow the rescue.
    uint32_t nt = tb == 0u ? kEveryRowKey : tb, nid = 0xFFFFFFFFu;
    if (over) {
      nt = tu;
      if (eligible >= A.k) {
        const uint64_t kth = select_top_each(each, A.k, S).prefix;
        if ((uint32_t)(kth >> 32) >= nt) {
          nt = (uint32_t)(kth >> 32);
          nid = composite_id(kth);
        }
      }
    }
    if (t == 0) queue_rescue(A, q, nt, nid, false);
    return;
  }
  const int r = (int)min<int64_t>(eligible, A.k);
  if (r > 0) {
    if (c <= A.cache_n) {
      // each thread copies its own segment to its place in the cache
      uint32_t j = so.x;
      each([&](uint64_t key) { cache[j++] = key; });
      __syncthreads();
      if (c <= kSortAll && c <= 4 * (int64_t)A.k) {
        // a short list: one sort of every candidate (excluded ones, key 0, sink to the end)
        bitonic_sort_desc(cache, (int)c);
        write_out(A, q, cache, r);
        return;
      }
      auto get = [&](int64_t i) { return cache[i]; };
      Sel64 sel{0ull, 0ull};
      if (c > r) sel = select_top(get, c, r, S);
      gather_sort(get, c, r, sel, sel_buf, &S.hist[0]);
    } else {
      // a list longer than the cache: each pass reads the segments again
      Sel64 sel{0ull, 0ull};
      if (c > r) sel = select_top_each(each, r, S);
      gather_sort_each(each, r, sel, sel_buf, &S.hist[0]);
    }
  }
  write_out(A, q, sel_buf, r);
}

template <int CT, int D>
static void launch_select(const SelectArgs& S, int grid, int round, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)final_select_kernel<CT, D>,
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              kSelCacheMax * (int)sizeof(uint64_t));
    attr = true;
  }
  hipLaunchKernelGGL((final_select_kernel<CT, D>), dim3(grid), dim3(kSelThreads),
                     (size_t)S.cache_n * sizeof(uint64_t), s, S, round);
}

// ------------------------------------------------------------------- planning
struct Plan {
  int b, b32, k, d, qdt, cdt;
  int nt;                    // masks of a multi-mask pass (0: one result set)
  int bv, bv32;              // lists: b per mask (virtual queries), and rounded up to 32
  int64_t excl_rw;           // exclusion words per query (0: one shared bitmap)
  int64_t n, n32, lo, blk0;  // rows [lo, n); n32 blocks from blk0
  int rm, rm_main, nqf, nqblk, G, rest, nseg;  // blocks per stage: sample/dense, main
  bool dense;
  int64_t capw;  // candidate entries per list segment
  size_t off_qtile, off_qexp, off_thr, off_thrb, off_ovf, off_thrid, off_rtail, off_nfail,
      off_flist, off_segcnt, off_del, off_cand, fixed;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Segments per query list: one per corpus slice of a pass (at most one slice per CU).
static int list_segments() { return std::min(device_cu_count(), kMaxSegments); }

// Default candidate capacity per query: 16 K, at least 32768, at most the corpus, spread
// over the segments.
static int64_t default_capw(int64_t n32, int k, int nseg) {
  const int64_t want = std::min<int64_t>(n32 * kFrag, std::max<int64_t>(16 * (int64_t)k, 32768));
  return (want + nseg - 1) / nseg;
}

// Rank of the estimated threshold among the G delegates: the sample holds a fraction
// f = G / n32 of the blocks, so about r / f items of the corpus reach the r-th delegate.
// r = c K f with c = 1 + 6 / sqrt(K f) keeps the chance that fewer than K items do (a
// rescue) far below one in a million for a random sample.
static int estimate_rank(int64_t n32, int G, int k) {
  if ((int64_t)G >= n32) return k;
  const double kf = (double)k * (double)G / (double)n32;
  const double c = 1.0 + 6.0 / std::sqrt(kf);
  const int r = (int)std::ceil(c * kf);
  return std::max(1, std::min(k, r));
}

// Most blocks a sample takes for `lists32` lists (rounded up to 32): kMaxSample, or up to four
// times that while the sample's block-list work stays within 2^25 blocks x lists. The larger
// sample tightens the estimate where the K best items are few in kMaxSample blocks (a large K
// against a large corpus) and every surplus survivor costs the main pass a slow-path walk: at
// N=10^8, D=64, B=1024, K=1000 the main pass took 10.44 instead of 10.97 ms with 32768 blocks.
static int64_t sample_cap(int lists32) {
  return std::max<int64_t>(kMaxSample, std::min<int64_t>(4 * (int64_t)kMaxSample, (int64_t{1} << 25) / lists32));
}

// capq: candidate capacity per query (< 0: the default).
// The pass covers rows [lo, n): the blocks from lo / 32 to the one holding row n - 1.
static void make_plan(Plan& p, int b, int64_t n, int d, int k, int qdt, int cdt, int64_t capq,
                      int64_t lo = 0, int nt = 0) {
  p.b = b;
  p.nt = nt;
  p.bv = b * std::max(nt, 1);
  p.bv32 = (p.bv + 31) / 32 * 32;
  p.excl_rw = 0;
  p.b32 = (b + 31) / 32 * 32;
  p.k = k;
  p.d = d;
  p.qdt = qdt;
  p.cdt = cdt;
  p.n = n;
  p.lo = lo;
  p.blk0 = lo / 32;
  p.n32 = (n + 31) / 32 - p.blk0;
  p.rm = stage_frags(cdt, d);
  p.rm_main = main_frags(cdt, d);
  int nqf_max = nt > 0 ? kMaskNqfMax : 16;
  while (nqf_max > 1 && !nqf_fits(cdt, d, nqf_max, nt > 0 ? kMaxMasks : 0)) nqf_max >>= 1;
  const int need = p.b32 / 32;
  int nqblk = (need + nqf_max - 1) / nqf_max;
  const int per = (need + nqblk - 1) / nqblk;
  p.nqf = 1;
  while (p.nqf < per) p.nqf <<= 1;
  p.nqblk = (need + p.nqf - 1) / p.nqf;
  p.nseg = list_segments();
  p.capw = capq < 0 ? default_capw(p.n32, k, p.nseg) : capq / p.nseg;
  p.dense = p.n32 < 2 * (int64_t)k + 64 && p.n32 * kFrag <= p.nseg * p.capw;
  // sampled blocks: a 16th of the corpus (the sample pass re-reads them), but no more than
  // needed for about 12 of the K best items to be expected in the sample (K G / n32 = 12,
  // where the margin c of estimate_rank is 2.73). Every survivor of the main pass costs it a
  // slow-path walk, so a larger sample shortens that pass; beyond about 12 items the sample
  // pass costs more than the main pass saves. At least 4 K, so that the K-th delegate usually
  // exists; at most sample_cap.
  const int64_t g12 = (12 * p.n32 + k - 1) / k;
  p.G = p.dense ? 0
                : (int)std::min<int64_t>(std::min<int64_t>(p.n32, sample_cap(p.bv32)),
                                         std::max<int64_t>(std::min<int64_t>(p.n32 / 16, g12), 4 * (int64_t)k));
  p.rest = p.dense ? 0 : estimate_rank(p.n32, p.G, k);
  const int E = elem_bytes(cdt);
  size_t o = 0;
  // first: the rescue queue count and the rescan count (bytes 0..7 of the workspace)
  p.off_nfail = o;
  o = align256(o + 8);
  p.off_qtile = o;
  o = align256(o + (size_t)p.b32 * d * E);
  p.off_qexp = o;
  o = align256(o + (size_t)p.b32 * 4);
  // per list (query, or virtual query of a multi-mask pass)
  p.off_thr = o;
  o = align256(o + (size_t)p.bv * 4);
  p.off_thrb = o;
  o = align256(o + (size_t)p.bv * 4);
  p.off_ovf = o;
  o = align256(o + (size_t)p.bv * 4);
  p.off_thrid = o;
  o = align256(o + (size_t)p.bv * 4);
  p.off_rtail = o;
  o = align256(o + (size_t)p.bv * 4);
  p.off_flist = o;
  o = align256(o + (size_t)p.bv * 4);
  p.off_segcnt = o;
  o = align256(o + (size_t)p.bv * p.nseg * 4);
  p.off_del = o;
  const int64_t gmax = std::max(p.G, 1);  // ranges plan over fewer rows, so no larger sample
  const int64_t tgroups = ((gmax + p.rm - 1) / p.rm + 15) / 16;
  o = align256(o + (size_t)tgroups * 16 * p.rm * (nt > 0 ? p.bv32 : p.b32) * 4);
  p.off_cand = o;
  p.fixed = o;
}

template <int CT, int D, int NT>
static int run_topk(const Plan& p, const void* queries, const void* corpus, const float* row_scale,
                    const uint32_t* exclude, const uint32_t* masks, int64_t mask_words,
                    float* out_scores, int32_t* out_ids, uint8_t* ws, hipStream_t s) {
  uint8_t* qtile = ws + p.off_qtile;
  int* qexp = (int*)(ws + p.off_qexp);
  uint32_t* thr = (uint32_t*)(ws + p.off_thr);
  uint32_t* thrb = (uint32_t*)(ws + p.off_thrb);
  uint32_t* ovf = (uint32_t*)(ws + p.off_ovf);
  uint32_t* segcnt = (uint32_t*)(ws + p.off_segcnt);
  uint32_t* nfail = (uint32_t*)(ws + p.off_nfail);
  uint32_t* flist = (uint32_t*)(ws + p.off_flist);
  uint32_t* del = (uint32_t*)(ws + p.off_del);
  uint64_t* cand = (uint64_t*)(ws + p.off_cand);
  uint32_t* thr_id = (uint32_t*)(ws + p.off_thrid);
  uint32_t* rtail = (uint32_t*)(ws + p.off_rtail);

  // A sampled pass over a bf16 or f32 index builds the operand tile in its sample pass (no
  // query scale to compute there); otherwise the prep kernel builds it.
  const bool fused_prep = !p.dense && fused_prep_ok(CT, D, p.nqf);
  int rc = MIPS_OK;
  if (!fused_prep) {
    if (p.qdt == MIPS_F32)
      hipLaunchKernelGGL((prep_queries_kernel<CT, MIPS_F32, D>), dim3(p.b32 / 32 * chunks_per_block(CT, D)), dim3(64), 0, s,
                         queries, p.b, qtile, qexp, ovf, p.bv, nfail);
    else
      hipLaunchKernelGGL((prep_queries_kernel<CT, MIPS_BF16, D>), dim3(p.b32 / 32 * chunks_per_block(CT, D)), dim3(64), 0, s,
                         queries, p.b, qtile, qexp, ovf, p.bv, nfail);
    if ((rc = check_launch())) return rc;
  }

  ScoreArgs A{};
  A.corpus = (const uint8_t*)corpus;
  A.row_scale = row_scale;
  // the score passes apply a shared bitmap as they read the corpus; one bitmap per query
  // is applied to each query's candidates by the final select
  A.exclude = p.excl_rw > 0 ? nullptr : exclude;
  A.qtile = qtile;
  A.qexp = qexp;
  A.n = p.n;
  A.lo = p.lo;
  A.blk0 = p.blk0;
  A.n32 = p.n32;
  A.b = p.b;
  A.b32 = p.b32;
  A.nqblk = p.nqblk;
  A.thr = thr;
  A.segcnt = segcnt;
  A.ovf = ovf;
  A.cand = cand;
  A.capw = p.capw;
  A.nseg = p.nseg;
  A.del = del;
  A.masks = masks;
  A.mask_words = mask_words;
  A.nmask = p.nt;
  A.bv32 = p.bv32;

  const int cus = device_cu_count();
  auto slices_for = [&](int64_t ntiles, int nqblk) {
    int64_t want = std::max<int64_t>(1, std::min(cus, p.nseg) / nqblk);
    if (want >= 8) want = want / 8 * 8;
    return (int)std::max<int64_t>(1, std::min<int64_t>(ntiles, want));
  };

  SelectArgs S{};
  S.corpus = (const uint8_t*)corpus;
  S.row_scale = row_scale;
  S.exclude = exclude;
  S.excl_rw = p.excl_rw;
  S.qtile = qtile;
  S.qexp = qexp;
  S.n = p.n;
  S.lo = p.lo;
  S.b = p.bv;
  S.k = p.k;
  S.cache_n = sel_cache_entries(p.k);
  S.masks = masks;
  S.mask_words = mask_words;
  S.breal = NT > 0 ? p.b : 0;
  S.capw = p.capw;
  S.nseg = p.nseg;
  S.thr = thr;
  S.thrb = thrb;
  S.thr_id = thr_id;
  S.rtail = rtail;
  S.segcnt = segcnt;
  S.ovf = ovf;
  S.cand = cand;
  S.nfail = nfail;
  S.flist = flist;
  S.out_scores = out_scores;
  S.out_ids = out_ids;

  hipEvent_t ev0, ev1;
  timing_events(&ev0, &ev1);

  if (p.dense) {
    A.nfrag = p.n32;
    A.ntiles = (p.n32 + p.rm - 1) / p.rm;
    A.nslices = slices_for(A.ntiles, p.nqblk);
    if ((rc = launch_score_nqf<CT, D, MODE_DENSE, NT>(p.nqf, A, A.nslices * p.nqblk, s, ev0, ev1))) return rc;
    S.dense_count = p.n32 * kFrag;
    launch_select<CT, D>(S, p.bv, 0, s);
    return check_launch();
  }

  // sample pass and thresholds
  A.nfrag = p.G;
  A.sample_step = ((uint64_t)p.n32 << 32) / (uint64_t)p.G;
  A.ntiles = (p.G + p.rm - 1) / p.rm;
  A.nslices = slices_for(A.ntiles, p.nqblk);
  if (fused_prep) {
    A.qraw = queries;
    A.qraw_f32 = p.qdt == MIPS_F32;
    A.nflags = p.bv;
    A.nfail = nfail;
  }
  if ((rc = launch_score_nqf<CT, D, MODE_SAMPLE, NT>(p.nqf, A, A.nslices * p.nqblk, s))) return rc;
  A.qraw = nullptr;
  hipLaunchKernelGGL(sample_threshold_kernel, dim3(p.bv), dim3(kSelThreads), 0, s, del, (int)A.ntiles,
                     p.rm, NT > 0 ? p.bv32 : p.b32, p.bv, p.k, p.rest, thr, thrb);
  if ((rc = check_launch())) return rc;

  // main pass
  A.nfrag = p.n32;
  A.ntiles = (p.n32 + p.rm_main - 1) / p.rm_main;
  A.nslices = slices_for(A.ntiles, p.nqblk);
  if ((rc = launch_score_nqf<CT, D, MODE_MAIN, NT>(p.nqf, A, A.nslices * p.nqblk, s, ev0, ev1))) return rc;
  S.dense_count = 0;
  S.nseg_used = A.nslices;
  launch_select<CT, D>(S, p.bv, 0, s);
  if ((rc = check_launch())) return rc;

  // rescue pass over the queued queries (one workgroup per slice loops over them)
  ScoreArgs R = A;
  R.qlist = flist;
  R.nlist = nfail;
  R.thr_id = thr_id;
  R.rtail = rtail;
  R.nqblk = 1;
  R.nslices = slices_for(A.ntiles, 1);
  if ((rc = launch_score_nqf<CT, D, MODE_MAIN, NT>(p.nqf, R, R.nslices, s))) return rc;
  S.nseg_used = R.nslices;
  launch_select<CT, D>(S, p.bv, 1, s);
  return check_launch();
}

template <int CT>
static int dispatch_d(const Plan& p, const void* queries, const void* corpus,
                      const float* row_scale, const uint32_t* exclude, const uint32_t* masks,
                      int64_t mask_words, float* out_scores, int32_t* out_ids, uint8_t* ws,
                      hipStream_t s) {
#define MIPS_RUN(DD)                                                                           \
  return p.nt > 0 ? run_topk<CT, DD, kMaxMasks>(p, queries, corpus, row_scale, exclude, masks, \
                                                mask_words, out_scores, out_ids, ws, s)        \
                  : run_topk<CT, DD, 0>(p, queries, corpus, row_scale, exclude, masks,         \
                                        mask_words, out_scores, out_ids, ws, s)
  switch (p.d) {
    case 16: if constexpr (CT != MIPS_FP8_E4M3 && CT != MIPS_INT8) { MIPS_RUN(16); } break;
    case 32: if constexpr (CT != MIPS_FP8_E4M3) { MIPS_RUN(32); } break;
    case 64: MIPS_RUN(64);
    case 128: MIPS_RUN(128);
    case 256: if constexpr (CT != MIPS_F32) { MIPS_RUN(256); } break;
  }
#undef MIPS_RUN
  return MIPS_ERR_UNSUPPORTED;
}

static int validate_topk(int32_t qdt, int32_t b, int32_t cdt, int64_t n, int32_t d, int32_t k) {
  if (qdt != MIPS_F32 && qdt != MIPS_BF16) return MIPS_ERR_UNSUPPORTED;
  if (cdt != MIPS_F32 && cdt != MIPS_BF16 && cdt != MIPS_FP8_E4M3 && cdt != MIPS_INT8)
    return MIPS_ERR_UNSUPPORTED;
  if (cdt == MIPS_F32 && qdt != MIPS_F32) return MIPS_ERR_UNSUPPORTED;
  if (b < 1 || n < 1 || n > (int64_t)0x7FFFFFFF - 64 || k < 1) return MIPS_ERR_INVALID_ARG;
  if (k > MIPS_K_MAX || b > MIPS_B_MAX) return MIPS_ERR_UNSUPPORTED;
  if (!corpus_d_supported(cdt, d)) return MIPS_ERR_UNSUPPORTED;
  return MIPS_OK;
}

static_assert(kMaxMasks == MIPS_MAX_MASKS, "the header's mask limit is the kernel's");

// Validation shared by every top-k entry point (no HIP call; the workspace is checked by
// topk_entry).
int validate_entry(const void* queries, int32_t query_dtype, int32_t b, const void* corpus,
                   const float* row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
                   const uint32_t* exclude, int64_t exclude_row_words, const uint32_t* masks,
                   int32_t nmasks, int64_t mask_words, const int64_t* ranges, int32_t nranges,
                   int32_t k, const float* out_scores, const int32_t* out_ids) {
  if (!queries || !corpus || !out_scores || !out_ids || !ranges) return MIPS_ERR_INVALID_ARG;
  const int rc0 = validate_topk(query_dtype, b, corpus_dtype, n, d, k);
  if (rc0 != MIPS_OK) return rc0;
  if (nranges < 1) return MIPS_ERR_INVALID_ARG;
  for (int r = 0; r < nranges; ++r)
    if (ranges[2 * r] < 0 || ranges[2 * r] >= ranges[2 * r + 1] || ranges[2 * r + 1] > n)
      return MIPS_ERR_INVALID_ARG;
  if (exclude_row_words < 0 || (exclude_row_words > 0 && (!exclude || exclude_row_words < (n + 31) / 32)))
    return MIPS_ERR_INVALID_ARG;
  if (nmasks > 0 && (!masks || mask_words < (n + 31) / 32 || exclude || !aligned(masks, 4)))
    return MIPS_ERR_INVALID_ARG;
  if ((int64_t)b * std::max(nmasks, 1) > MIPS_B_MAX) return MIPS_ERR_UNSUPPORTED;
  if ((corpus_dtype == MIPS_FP8_E4M3 || corpus_dtype == MIPS_INT8) && !row_scale)
    return MIPS_ERR_INVALID_ARG;
  if (!aligned(queries, 4) || !aligned(corpus, 16) || !aligned(out_scores, 4) ||
      !aligned(out_ids, 4) || (exclude && !aligned(exclude, 4)) ||
      (row_scale && !aligned(row_scale, 4)))
    return MIPS_ERR_INVALID_ARG;
  return MIPS_OK;
}

// Every top-k entry point: validation, then one pass per id range (nmasks > 0: one
// multi-mask pass over the whole corpus, lists per (mask, query)).
int topk_entry(const void* queries, int32_t query_dtype, int32_t b, const void* corpus,
               const float* row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
               const uint32_t* exclude, int64_t exclude_row_words, const uint32_t* masks,
               int32_t nmasks, int64_t mask_words, const int64_t* ranges, int32_t nranges,
               int32_t k, float* out_scores, int32_t* out_ids, void* workspace,
               size_t workspace_bytes, void* stream) {
  const int rcv = validate_entry(queries, query_dtype, b, corpus, row_scale, corpus_dtype, n, d,
                                 exclude, exclude_row_words, masks, nmasks, mask_words, ranges,
                                 nranges, k, out_scores, out_ids);
  if (rcv != MIPS_OK) return rcv;
  if (!workspace || !aligned(workspace, 256)) return MIPS_ERR_INVALID_ARG;
  // the whole corpus's plan bounds every range's fixed part and capacity
  Plan p;
  make_plan(p, b, n, d, k, query_dtype, corpus_dtype, -1, 0, nmasks);
  if (workspace_bytes < p.fixed) return MIPS_ERR_WORKSPACE;
  // candidate capacity per list: whole segments of what the workspace holds
  const int64_t capq = (int64_t)((workspace_bytes - p.fixed) / ((size_t)p.bv * 8u));
  if (capq / p.nseg < 1) return MIPS_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  for (int r = 0; r < nranges; ++r) {
    make_plan(p, b, ranges[2 * r + 1], d, k, query_dtype, corpus_dtype, capq, ranges[2 * r], nmasks);
    p.excl_rw = exclude_row_words;
    float* os = out_scores + (int64_t)r * p.bv * k;
    int32_t* oi = out_ids + (int64_t)r * p.bv * k;
    int rc;
    switch (corpus_dtype) {
      case MIPS_F32:
        rc = dispatch_d<MIPS_F32>(p, queries, corpus, row_scale, exclude, masks, mask_words, os, oi, ws, s);
        break;
      case MIPS_BF16:
        rc = dispatch_d<MIPS_BF16>(p, queries, corpus, row_scale, exclude, masks, mask_words, os, oi, ws, s);
        break;
      case MIPS_INT8:
        rc = dispatch_d<MIPS_INT8>(p, queries, corpus, row_scale, exclude, masks, mask_words, os, oi, ws, s);
        break;
      default:
        rc = dispatch_d<MIPS_FP8_E4M3>(p, queries, corpus, row_scale, exclude, masks, mask_words, os, oi, ws, s);
        break;
    }
    if (rc != MIPS_OK) return rc;
  }
  return MIPS_OK;
}

size_t workspace_bytes_for(int32_t b, int64_t n, int32_t d, int32_t k, int32_t qdt,
                           int32_t cdt, int32_t nmasks, int64_t candidates) {
  if (validate_topk(qdt, b, cdt, n, d, k) != MIPS_OK) return 0;
  if (nmasks < 0 || nmasks > kMaxMasks || (int64_t)b * std::max(nmasks, 1) > MIPS_B_MAX) return 0;
  Plan p;
  make_plan(p, b, n, d, k, qdt, cdt, -1, 0, nmasks);
  const int64_t capw = candidates < 0 ? p.capw : (candidates + p.nseg - 1) / p.nseg;
  return p.fixed + (size_t)p.bv * (size_t)p.nseg * (size_t)capw * 8u;
}

}  // namespace mips

extern "C" {

size_t mips_topk_workspace_size(int32_t b, int64_t n, int32_t d, int32_t k, int32_t query_dtype,
                                int32_t corpus_dtype) {
  return mips::workspace_bytes_for(b, n, d, k, query_dtype, corpus_dtype, 0, -1);
}

size_t mips_topk_workspace_size_for(int32_t b, int64_t n, int32_t d, int32_t k, int32_t query_dtype,
                                    int32_t corpus_dtype, int64_t candidates_per_query) {
  if (candidates_per_query < 1) return 0;
  return mips::workspace_bytes_for(b, n, d, k, query_dtype, corpus_dtype, 0, candidates_per_query);
}

size_t mips_topk_masks_workspace_size(int32_t b, int64_t n, int32_t d, int32_t k, int32_t query_dtype,
                                      int32_t corpus_dtype, int32_t nmasks,
                                      int64_t candidates_per_list) {
  if (nmasks < 1) return 0;
  return mips::workspace_bytes_for(b, n, d, k, query_dtype, corpus_dtype, nmasks,
                                   candidates_per_list < 1 ? -1 : candidates_per_list);
}

int mips_topk(const void* queries, int32_t query_dtype, int32_t b, const void* corpus,
              const float* row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
              const uint32_t* exclude, int64_t exclude_row_words, int32_t k, float* out_scores,
              int32_t* out_ids, void* workspace, size_t workspace_bytes, void* stream) {
  const int64_t whole[2] = {0, n};
  return mips::topk_entry(queries, query_dtype, b, corpus, row_scale, corpus_dtype, n, d, exclude,
                          exclude_row_words, nullptr, 0, 0, whole, 1, k, out_scores, out_ids,
                          workspace, workspace_bytes, stream);
}

int mips_topk_ranges(const void* queries, int32_t query_dtype, int32_t b, const void* corpus,
                     const float* row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
                     const uint32_t* exclude, int64_t exclude_row_words, const int64_t* ranges,
                     int32_t nranges, int32_t k, float* out_scores, int32_t* out_ids,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return mips::topk_entry(queries, query_dtype, b, corpus, row_scale, corpus_dtype, n, d, exclude,
                          exclude_row_words, nullptr, 0, 0, ranges, nranges, k, out_scores,
                          out_ids, workspace, workspace_bytes, stream);
}

int mips_topk_masks(const void* queries, int32_t query_dtype, int32_t b, const void* corpus,
                    const float* row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
                    const uint32_t* masks, int32_t nmasks, int64_t mask_words, int32_t k,
                    float* out_scores, int32_t* out_ids, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (nmasks < 1 || nmasks > mips::kMaxMasks) return nmasks < 1 ? MIPS_ERR_INVALID_ARG : MIPS_ERR_UNSUPPORTED;
  const int64_t whole[2] = {0, n};
  return mips::topk_entry(queries, query_dtype, b, corpus, row_scale, corpus_dtype, n, d, nullptr,
                          0, masks, nmasks, mask_words, whole, 1, k, out_scores, out_ids,
                          workspace, workspace_bytes, stream);
}

}  // extern "C"
