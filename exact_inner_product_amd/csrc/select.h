// select.h -- block-wide radix selection and sorting of 64-bit keys in LDS (gfx950).
//
// Every helper here is called by all kSelThreads (= 256) threads of a workgroup.
#pragma once

#include "common.h"
#include "../../include/mips.h"

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

// The r largest of the workgroup's keys (1 <= r <= their number), MSD radix select with
// 8-bit digits starting at the highest bit where the keys differ; stops as soon as the
// boundary bin holds exactly the remaining rank. With distinct keys exactly r keys satisfy
// the returned test; with ties, prefix is still a lower bound of the r-th largest key.
// each(f) calls f(key) for every key the calling thread holds; the keys must be the same
// on every call.
template <typename Each>
__device__ Sel64 select_top_each(Each each, int r, SelScratch& S) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint64_t lo = ~0ull, hi = 0ull;
  each([&](uint64_t k) {
    lo = k < lo ? k : lo;
    hi = k > hi ? k : hi;
  });
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
    each([&](uint64_t k) {
      if ((k & mask) == prefix) atomicAdd(&S.hist[(k >> lb) & dmask], 1u);
    });
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

// The r largest of n keys get(0 .. n-1), thread t taking i = t, t + kSelThreads, ...
template <typename Get>
__device__ Sel64 select_top(Get get, int64_t n, int r, SelScratch& S) {
  return select_top_each(
      [&](auto f) {
        for (int64_t i = threadIdx.x; i < n; i += kSelThreads) f(get(i));
      },
      r, S);
}

__device__ __forceinline__ int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

__device__ __forceinline__ void cmp_swap_desc(uint64_t& a, uint64_t& b, bool desc) {
  const bool sw = desc ? a < b : a > b;
  const uint64_t x = a;
  a = sw ? b : a;
  b = sw ? x : b;
}

// Sorts s[0..r) descending in place, r <= P (P a power of two, 2 <= P <= MIPS_K_MAX), as
// a bitonic network held in registers and fully unrolled: element e = t + kSelThreads * h
// lives in thread t, slot h. Partners less than a wave apart are exchanged by constant
// shuffles, partners in another slot of the same thread in registers, and only the strides
// of at least a wave and less than kSelThreads go through LDS (with barriers).
template <int P>
__device__ void bitonic_sort_desc_p(uint64_t* s, int r) {
  constexpr int kPer = (P + kSelThreads - 1) / kSelThreads;
  const int t = threadIdx.x;
  uint64_t x[kPer];
#pragma unroll
  for (int h = 0; h < kPer; ++h) {
    const int e = t + kSelThreads * h;
    x[h] = (e < r) ? s[e] : 0ull;  // padding (0) sinks to the end
  }
  __syncthreads();
#pragma unroll
  for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= kSelThreads) {
        const int hs = stride / kSelThreads;
#pragma unroll
        for (int h = 0; h < kPer; ++h) {
          if ((h & hs) == 0) {
            const int e = t + kSelThreads * h;
            cmp_swap_desc(x[h], x[h | hs], (e & size) == 0);
          }
        }
      } else {
        uint64_t y[kPer];
        if (stride >= kWave) {
#pragma unroll
          for (int h = 0; h < kPer; ++h) s[t + kSelThreads * h] = x[h];
          __syncthreads();
#pragma unroll
          for (int h = 0; h < kPer; ++h) y[h] = s[(t ^ stride) + kSelThreads * h];
          __syncthreads();
        } else {
#pragma unroll
          for (int h = 0; h < kPer; ++h) y[h] = shfl_xor_u64(x[h], stride);
        }
#pragma unroll
        for (int h = 0; h < kPer; ++h) {
          const int e = t + kSelThreads * h;
          const bool keep_hi = ((e & stride) == 0) == ((e & size) == 0);
          const uint64_t hi = x[h] > y[h] ? x[h] : y[h];
          const uint64_t lo = x[h] > y[h] ? y[h] : x[h];
          x[h] = keep_hi ? hi : lo;
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kPer; ++h) {
    const int e = t + kSelThreads * h;
    if (e < r) s[e] = x[h];
  }
  __syncthreads();
}

__device__ inline void bitonic_sort_desc(uint64_t* s, int r) {
  if (r <= 64) bitonic_sort_desc_p<64>(s, r);
  else if (r <= 256) bitonic_sort_desc_p<256>(s, r);
  else if (r <= 512) bitonic_sort_desc_p<512>(s, r);
  else bitonic_sort_desc_p<1024>(s, r);
}

// Gathers the r selected keys (visited as by select_top_each) into out[0..r) and sorts
// them descending. The keys are distinct (composite keys carry the id).
template <typename Each>
__device__ void gather_sort_each(Each each, int r, Sel64 sel, uint64_t* out, uint32_t* cnt) {
  if (threadIdx.x == 0) *cnt = 0u;
  __syncthreads();
  each([&](uint64_t key) {
    if ((key & sel.mask) >= sel.prefix) {
      const uint32_t slot = atomicAdd(cnt, 1u);
      if (slot < (uint32_t)r) out[slot] = key;
    }
  });
  __syncthreads();
  bitonic_sort_desc(out, r);
}

template <typename Get>
__device__ void gather_sort(Get get, int64_t n, int r, Sel64 sel, uint64_t* out, uint32_t* cnt) {
  gather_sort_each(
      [&](auto f) {
        for (int64_t i = threadIdx.x; i < n; i += kSelThreads) f(get(i));
      },
      r, sel, out, cnt);
}

}  // namespace mips
