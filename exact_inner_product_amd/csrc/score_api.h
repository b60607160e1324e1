// score_api.h -- the fused score pass of mips_topk: shared constants, its argument block
// and the launcher that each per-(dtype, width) translation unit instantiates.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace mips {

constexpr int kStageCap = 512;      // staged survivors per wave
constexpr int kStageBurst = 256;    // room kept free before each stage
constexpr int kLdsLimit = 160 * 1024;
constexpr int kMaxSample = 8192;    // sampled 32-row blocks

constexpr int kMaxSegments = 256;   // list segments per query (corpus slices of a pass)
constexpr int kSimdStageBytes = 16384;  // corpus bytes per SIMD and pipeline stage
constexpr int kPipeStages = 3;      // corpus stages per wave: one in use, two in flight
constexpr int kSelCacheMax = 8192;  // candidates the final select caches in LDS, at most
constexpr int kMaxMasks = 4;        // result sets (exclusion masks) of one multi-mask pass
constexpr int kMaskNqfMax = 4;      // query fragments per workgroup of a multi-mask pass

// Passes of the score kernel: the main filter pass (also the rescue pass), the sample pass
// (delegates of a strided block sample) and the dense pass (every score, small corpora).
enum { MODE_MAIN = 0, MODE_SAMPLE = 1, MODE_DENSE = 2 };

// Corpus blocks per pipeline stage for `wps` waves per SIMD: 16 KiB of corpus per SIMD and
// stage, split between its waves (at most 4 blocks per wave with one wave, 2 with two). An
// int8 stage also holds 16 row scales per lane and block, so it takes half the bytes and at
// most 2 blocks.
__host__ __device__ constexpr int frags_for(int ct, int d, int wps) {
  const int cap = (ct == MIPS_INT8 || wps > 1) ? 2 : 4;
  const int bytes = kSimdStageBytes / wps / (ct == MIPS_INT8 ? 2 : 1);
  const int r = bytes / (int)block_bytes(ct, d);
  return r < 1 ? 1 : (r > cap ? cap : r);
}
// Registers a wave of the main pass needs, roughly: the stage ring, int8 row scales, two
// fragments' accumulators, the query operand and about 60 for addresses and the epilogue.
__host__ __device__ constexpr int score_regs(int ct, int d, int rm) {
  const int nch = chunks_per_block(ct, d);
  return kPipeStages * rm * nch * 4 + (ct == MIPS_INT8 ? kPipeStages * rm * 16 : 0) +
         2 * rm * 16 + nch * 4 + 60;
}
// Waves per SIMD of the score kernel. With one wave, its in-order issue stalls the matrix
// pipe whenever it waits (on an accumulator, an LDS read, a branch); a second wave fills
// those gaps. Two waves split the 512 registers, so the second wave is used where the
// pass fits in 256 (one 8 KiB block per stage, or two smaller ones).
__host__ __device__ constexpr int score_wps(int ct, int d) {
  return score_regs(ct, d, frags_for(ct, d, 2)) <= 240 ? 2 : 1;
}
__host__ __device__ constexpr int score_threads(int ct, int d) { return 256 * score_wps(ct, d); }
__host__ __device__ constexpr int score_waves(int ct, int d) { return 4 * score_wps(ct, d); }
__host__ __device__ constexpr int stage_frags(int ct, int d) {
  return frags_for(ct, d, score_wps(ct, d));
}
// Main pass with two blocks per stage. Where two waves share a SIMD with one block per
// stage, each query operand read from LDS feeds only one block's MFMAs, and LDS read
// bandwidth becomes a co-bound of the pass. The main pass then takes two blocks per stage
// in a two-stage ring (the same stage bytes in flight per SIMD) with one accumulator set
// per wave, which fits the 256 registers; the sample and dense passes keep one block.
__host__ __device__ constexpr bool main_doubles(int ct, int d) {
  // (f32 keeps its 3-stage ring; fp8 at D=256 reaches the 256 registers with one 4-byte
  // per-lane value spilled, a constant that only the slow path reloads)
  return ct != MIPS_F32 && score_wps(ct, d) == 2 && stage_frags(ct, d) == 1 &&
         2 * 2 * chunks_per_block(ct, d) * 4 + (ct == MIPS_INT8 ? 2 * 2 * 16 : 0) + 2 * 16 +
                 chunks_per_block(ct, d) * 4 + 60 <= 256;
}
__host__ __device__ constexpr int main_frags(int ct, int d) {
  return main_doubles(ct, d) ? 2 : stage_frags(ct, d);
}
// The sample pass builds the query operand tile itself (no separate prep kernel) for a bf16
// or f32 index, where that takes no per-query scale, with two waves per SIMD and at most
// 8 query fragments (beyond that the fill's registers would spill in the sample pass).
__host__ __device__ constexpr bool fused_prep_ok(int ct, int d, int nqf) {
  return (ct == MIPS_BF16 || ct == MIPS_F32) && score_wps(ct, d) == 2 && nqf <= 8;
}
// LDS of a score workgroup holding 32 * nqf queries: the query tile, 16 bytes of per-column
// state per query and the survivor staging of every wave (8-byte key, 2-byte column). A
// multi-mask pass (nt masks) adds a threshold and a survivor counter per column and mask.
__host__ __device__ constexpr int score_lds_bytes(int ct, int d, int nqf, int nt = 0) {
  return kFrag * nqf * (d * elem_bytes(ct) + 16 + 8 * nt) + score_waves(ct, d) * kStageCap * (8 + 2);
}
__host__ __device__ constexpr bool nqf_fits(int ct, int d, int nqf, int nt = 0) {
  return score_lds_bytes(ct, d, nqf, nt) <= kLdsLimit;
}
// Entries of the final select's LDS candidate cache for k results: room for about 8 k
// candidates (a longer list is read from memory on every pass over it), at least 2048 (the
// exact rescan compacts a buffer that holds k + 1024 keys) and at most kSelCacheMax. The
// smaller the cache, the more lists a compute unit selects at once.
__host__ __device__ constexpr int sel_cache_entries(int k) {
  int c = 2048;
  while (c < 8 * k && c < kSelCacheMax) c <<= 1;
  return c;
}

struct ScoreArgs {
  const uint8_t* corpus;
  const float* row_scale;
  const uint32_t* exclude;
  const uint8_t* qtile;
  const int* qexp;
  int64_t n;        // rows below n take part (the end of the id range)
  int64_t lo;       // rows at or above lo take part (the start of the id range)
  int64_t blk0;     // first block of the pass (lo / 32); block ids are absolute
  int64_t n32;      // 32-row blocks in the pass
  int64_t nfrag;    // blocks this pass covers: n32, or G sampled blocks (strided)
  int64_t ntiles;   // stage tiles of the pass
  int b;
  int b32;
  int nqblk;        // query blocks in the grid
  int nslices;      // corpus slices in the grid
  const uint32_t* thr;    // per-query threshold keys (0: query not scored here)
  // rescue pass: per-list id bound of a composite threshold (a row whose score equals the
  // list's threshold passes only with an id at or below it), and per-list survivor
  // counts; a rescued list is one contiguous run of nseg * capw entries, filled through
  // its count as an atomic tail
  const uint32_t* thr_id;
  uint32_t* rtail;
  uint32_t* segcnt;       // [b][nseg] survivors found per (query, segment)
  uint32_t* ovf;
  uint64_t* cand;         // [b][nseg][capw] candidate keys; dense pass: [b][nseg * capw]
  int64_t capw;           // entries per segment
  int nseg;               // segments per query (one per corpus slice)
  const uint32_t* qlist;  // rescue pass: queued query ids ...
  const uint32_t* nlist;  // ... and their number (device); NULL for the full batch
  uint32_t* del;          // sample delegates [tile/16][b32][16][RM]: one per block and query
  uint64_t sample_step;   // sampled block j is block (j * sample_step) >> 32
  // Multi-mask pass: nmask result sets, mask t excluding the rows whose bit is set in
  // masks[t * mask_words ..]; result set t of query q is the virtual query t * b + q, which
  // indexes thr, segcnt, ovf, cand and the rescue list (`exclude` is not used).
  const uint32_t* masks;
  int64_t mask_words;
  int nmask;
  int bv32;               // virtual queries rounded up to 32: the delegate stride
  // Sample pass over a bf16 or f32 index: the raw queries ([b, D], f32 if qraw_f32, else
  // bf16) from which each workgroup builds its operand tile; the slice-0 workgroup of each
  // query block also writes the tile to qtile for the later passes, and workgroup 0 clears
  // the per-list flags ovf[0, nflags) and *nfail. NULL: the tile is read from qtile.
  const void* qraw;
  int qraw_f32;
  int nflags;
  uint32_t* nfail;
};

// Launches score_kernel<CT, D, nqf, MODE, NT> (nqf in {1, 2, 4, 8, 16}; NT = 0 for one
// result set, kMaxMasks for a multi-mask pass); defined in score_inst.hip, built once per
// corpus dtype and width. With both events given, the dispatch records e0 at the kernel's
// start and e1 at its end.
template <int CT, int D, int MODE, int NT = 0>
int launch_score_nqf(int nqf, const ScoreArgs& A, int grid, hipStream_t s, hipEvent_t e0 = nullptr,
                     hipEvent_t e1 = nullptr);

}  // namespace mips
