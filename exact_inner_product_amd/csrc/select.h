// select.h -- block-wide radix selection and sorting of 64-bit keys in LDS (gfx950).
//
// Every helper here is called by all kSelThreads (= 256) threads of a workgroup.
#pragma once

#include "common.h"

namespace mips {

constexpr int kSelThreads = 256;

struct DigitPick {
  uint32_t digit, rem, bin;
};

// hist[0..255]: keys per digit value (under the current prefix). Finds the digit d with
// fewer than `rem` keys above it and at least `rem` at or above it, by a prefix sum over
// the bins taken from the top. Returns d, the rank left inside bin d and the bin's size.
__device__ inline DigitPick pick_digit(const uint32_t* hist, uint32_t rem, uint32_t* wsum,
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
__device__ inline void bitonic_desc(uint64_t* s, int p) {
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

// Gathers the r selected keys of `get` into out[0..r) and sorts them descending.
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

}  // namespace mips
