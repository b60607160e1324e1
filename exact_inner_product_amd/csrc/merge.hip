// merge.hip -- merge of several sorted per-query result lists into one top-k (gfx950).
//
// A small fresh index is searched beside the large base index and the two result lists
// are merged by score ("Two-Tower Retrieval at Industrial Scale", engineeringmaxxing.com,
// the fresh-shard pattern); the same merge joins the per-shard top-k lists of a corpus
// split across devices. The result is exact for its inputs: the union of the lists, ids
// shifted by each list's offset, cut to the best k by score descending, then id
// ascending.
#include "common.h"
#include "host.h"
#include "select.h"

namespace mips {

constexpr int kMergeMaxLists = 64;

struct MergeArgs {
  const float* in_s;     // [p, b, k_in]
  const int32_t* in_id;  // [p, b, k_in]; id < 0 is padding
  int p, b, k_in, k_out;
  float* out_s;          // [b, k_out]
  int32_t* out_id;
  int64_t off[kMergeMaxLists];
};

// One workgroup per query: the p * k_in entries are read as 64-bit composite keys
// (padding reads as 0, below every real key), the k_out largest are selected by the
// radix select and sorted.
__global__ __launch_bounds__(kSelThreads) void merge_topk_kernel(MergeArgs A) {
  __shared__ uint64_t sel_buf[MIPS_K_MAX];
  __shared__ SelScratch S;
  __shared__ int64_t off[kMergeMaxLists];
  __shared__ uint32_t nvalid;
  const int q = blockIdx.x;
  const int t = threadIdx.x;
  if (t < kMergeMaxLists) off[t] = t < A.p ? A.off[t] : 0;
  if (t == 0) nvalid = 0u;
  __syncthreads();
  const int64_t m = (int64_t)A.p * A.k_in;
  auto get = [&](int64_t i) -> uint64_t {
    const int l = (int)(i / A.k_in);
    const int64_t o = ((int64_t)l * A.b + q) * A.k_in + (i - (int64_t)l * A.k_in);
    const int32_t id = A.in_id[o];
    if (id < 0) return 0ull;
    return composite(score_key(A.in_s[o]), (uint32_t)(id + off[l]));
  };
  uint32_t mine = 0u;
  for (int64_t i = t; i < m; i += kSelThreads) mine += get(i) != 0ull;
  atomicAdd(&nvalid, mine);
  __syncthreads();
  const int r = (int)min<int64_t>((int64_t)nvalid, A.k_out);
  if (r > 0) {
    Sel64 sel{0ull, 0ull};
    if (m > r) sel = select_top(get, m, r, S);
    gather_sort(get, m, r, sel, sel_buf, &S.hist[0]);
  }
  for (int j = t; j < A.k_out; j += kSelThreads) {
    float sc = -INFINITY;
    int32_t id = -1;
    if (j < r) {
      sc = key_score((uint32_t)(sel_buf[j] >> 32));
      id = (int32_t)composite_id(sel_buf[j]);
    }
    A.out_s[(int64_t)q * A.k_out + j] = sc;
    A.out_id[(int64_t)q * A.k_out + j] = id;
  }
}

// ----------------------------------------------------------- multi-interest merge
// A user with m interest vectors scores an item by its best match over them (the max of
// "Two-Tower Retrieval at Industrial Scale", section "Beyond Dot Products": K interest
// vectors, K searches, results merged). Each interest's own top-k list is merged per user:
// an id that several interests return keeps its highest score, then the best k_out ids are
// kept. When every list is its interest's exact top-k_out, the result is the exact top-k_out
// by max score (an item in the max-score top-k is in the top-k of its best interest).
constexpr int kInterestEntries = 2048;  // m * k_in per user
constexpr int kInterestHash = 4096;     // open-addressing table, load at most 1/2
constexpr uint32_t kEmptyId = 0xFFFFFFFFu;

struct InterestArgs {
  const float* in_s;     // [b, m, k_in]
  const int32_t* in_id;  // [b, m, k_in]; id < 0 is padding
  int b, m, k_in, k_out;
  float* out_s;          // [b, k_out]
  int32_t* out_id;
};

__global__ __launch_bounds__(kSelThreads) void merge_interests_kernel(InterestArgs A) {
  __shared__ uint32_t hid[kInterestHash];
  __shared__ uint32_t hkey[kInterestHash];
  __shared__ uint64_t sel_buf[MIPS_K_MAX];
  __shared__ SelScratch S;
  __shared__ uint32_t nvalid;
  const int q = blockIdx.x;
  const int t = threadIdx.x;
  for (int i = t; i < kInterestHash; i += kSelThreads) {
    hid[i] = kEmptyId;
    hkey[i] = 0u;
  }
  if (t == 0) nvalid = 0u;
  __syncthreads();
  const int64_t base = (int64_t)q * A.m * A.k_in;
  const int m = A.m * A.k_in;
  for (int e = t; e < m; e += kSelThreads) {
    const int32_t id = A.in_id[base + e];
    if (id < 0) continue;
    const uint32_t key = score_key(A.in_s[base + e]);
    uint32_t slot = ((uint32_t)id * 2654435761u) & (kInterestHash - 1);  // Knuth's multiplier
    for (;;) {  // at most m < kInterestHash distinct ids: a free or matching slot exists
      const uint32_t prev = atomicCAS(&hid[slot], kEmptyId, (uint32_t)id);
      if (prev == kEmptyId || prev == (uint32_t)id) {
        atomicMax(&hkey[slot], key);
        break;
      }
      slot = (slot + 1u) & (kInterestHash - 1);
    }
  }
  __syncthreads();
  auto get = [&](int64_t i) -> uint64_t {
    return hid[i] == kEmptyId ? 0ull : composite(hkey[i], hid[i]);
  };
  uint32_t mine = 0u;
  for (int i = t; i < kInterestHash; i += kSelThreads) mine += hid[i] != kEmptyId;
  atomicAdd(&nvalid, mine);
  __syncthreads();
  const int r = (int)min<uint32_t>(nvalid, (uint32_t)A.k_out);
  if (r > 0) {
    Sel64 sel{0ull, 0ull};
    if (kInterestHash > r) sel = select_top(get, kInterestHash, r, S);
    gather_sort(get, kInterestHash, r, sel, sel_buf, &S.hist[0]);
  }
  for (int j = t; j < A.k_out; j += kSelThreads) {
    float sc = -INFINITY;
    int32_t id = -1;
    if (j < r) {
      sc = key_score((uint32_t)(sel_buf[j] >> 32));
      id = (int32_t)composite_id(sel_buf[j]);
    }
    A.out_s[(int64_t)q * A.k_out + j] = sc;
    A.out_id[(int64_t)q * A.k_out + j] = id;
  }
}

// ------------------------------------------------------------------ type masks
// Bitmap of the ids a type-restricted search must skip: id i is excluded when its type is
// not the target (the per-type mask of `RecsysTwoTowerModel.forward`, dataset_types ==
// target) or when the base bitmap excludes it. One thread per 32-id word.
__global__ __launch_bounds__(256) void type_bitmap_kernel(const int32_t* __restrict__ types,
                                                          int64_t n, int32_t target,
                                                          const uint32_t* __restrict__ base,
                                                          uint32_t* __restrict__ out) {
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= (n + 31) / 32) return;
  uint32_t bits = base ? base[w] : 0u;
  for (int r = 0; r < 32; ++r) {
    const int64_t i = w * 32 + r;
    if (i >= n || types[i] != target) bits |= 1u << r;
  }
  out[w] = bits;
}

}  // namespace mips

extern "C" {

int mips_type_bitmap(const int32_t* item_types, int64_t n, int32_t target,
                     const uint32_t* exclude, uint32_t* out_bitmap, void* stream) {
  if (!item_types || !out_bitmap || n < 1) return MIPS_ERR_INVALID_ARG;
  if (!mips::aligned(item_types, 4) || !mips::aligned(out_bitmap, 4) ||
      (exclude && !mips::aligned(exclude, 4)))
    return MIPS_ERR_INVALID_ARG;
  const int64_t words = (n + 31) / 32;
  const int64_t grid = (words + 255) / 256;
  if (grid > 0x7FFFFFFF) return MIPS_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mips::type_bitmap_kernel, dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)stream, item_types, n, target, exclude, out_bitmap);
  return mips::check_launch();
}


int mips_merge_interests(const float* in_scores, const int32_t* in_ids, int32_t b, int32_t m,
                         int32_t k_in, int32_t k_out, float* out_scores, int32_t* out_ids,
                         void* stream) {
  if (!in_scores || !in_ids || !out_scores || !out_ids) return MIPS_ERR_INVALID_ARG;
  if (b < 1 || m < 1 || k_in < 1 || k_out < 1) return MIPS_ERR_INVALID_ARG;
  if (k_out > MIPS_K_MAX || b > MIPS_B_MAX || (int64_t)m * k_in > mips::kInterestEntries)
    return MIPS_ERR_UNSUPPORTED;
  if (!mips::aligned(in_scores, 4) || !mips::aligned(in_ids, 4) || !mips::aligned(out_scores, 4) ||
      !mips::aligned(out_ids, 4))
    return MIPS_ERR_INVALID_ARG;
  mips::InterestArgs A{in_scores, in_ids, b, m, k_in, k_out, out_scores, out_ids};
  hipLaunchKernelGGL(mips::merge_interests_kernel, dim3(b), dim3(mips::kSelThreads), 0,
                     (hipStream_t)stream, A);
  return mips::check_launch();
}

int mips_merge_topk(const float* in_scores, const int32_t* in_ids, const int64_t* offsets,
                    int32_t p, int32_t b, int32_t k_in, int32_t k_out, float* out_scores,
                    int32_t* out_ids, void* stream) {
  if (!in_scores || !in_ids || !offsets || !out_scores || !out_ids) return MIPS_ERR_INVALID_ARG;
  if (p < 1 || p > mips::kMergeMaxLists || b < 1 || k_in < 1 || k_out < 1)
    return MIPS_ERR_INVALID_ARG;
  if (k_out > MIPS_K_MAX || b > MIPS_B_MAX) return MIPS_ERR_UNSUPPORTED;
  if ((int64_t)p * k_in > 0x7FFFFFFF) return MIPS_ERR_INVALID_ARG;
  if (!mips::aligned(in_scores, 4) || !mips::aligned(in_ids, 4) || !mips::aligned(out_scores, 4) ||
      !mips::aligned(out_ids, 4))
    return MIPS_ERR_INVALID_ARG;
  mips::MergeArgs A{};
  for (int l = 0; l < p; ++l) {
    if (offsets[l] < 0 || offsets[l] > 0x7FFFFFFF) return MIPS_ERR_INVALID_ARG;
    A.off[l] = offsets[l];
  }
  A.in_s = in_scores;
  A.in_id = in_ids;
  A.p = p;
  A.b = b;
  A.k_in = k_in;
  A.k_out = k_out;
  A.out_s = out_scores;
  A.out_id = out_ids;
  hipLaunchKernelGGL(mips::merge_topk_kernel, dim3(b), dim3(mips::kSelThreads), 0,
                     (hipStream_t)stream, A);
  return mips::check_launch();
}

}  // extern "C"
