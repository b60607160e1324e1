// host.h -- host-side helpers of the libmips C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mips.h"

namespace mips {

// Records the HIP error of the last failed launch on this thread.
void set_last_hip_error(hipError_t e);

// Returns MIPS_OK, or records the launch error and returns MIPS_ERR_HIP.
inline int check_launch() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_last_hip_error(e);
    return MIPS_ERR_HIP;
  }
  return MIPS_OK;
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// A launch counts its work-items per grid dimension in 32 bits. Row-wise kernels of 256
// threads are split into launches of at most this many workgroups (2^30 work-items).
constexpr int64_t kMaxGridBlocks = int64_t(1) << 22;

inline bool corpus_d_supported(int dtype, int d) {
  if (dtype == MIPS_FP8_E4M3) return d == 64 || d == 128 || d == 256;
  if (dtype == MIPS_F32) return d == 16 || d == 32 || d == 64 || d == 128;
  if (dtype == MIPS_BF16) return d == 16 || d == 32 || d == 64 || d == 128 || d == 256;
  if (dtype == MIPS_INT8) return d == 32 || d == 64 || d == 128 || d == 256;
  return false;
}

// Compute units of the current device (cached per device).
int device_cu_count();

// Timing hook of mips_set_timing_events.
void timing_events(hipEvent_t* before, hipEvent_t* after);

// The top-k entry points' shared parts (topk.hip): argument validation without any HIP call;
// validation and the passes over a caller-given workspace; the workspace a call needs with
// `candidates` per list (< 0: the default capacity), 0 for unsupported arguments.
int validate_entry(const void* queries, int32_t query_dtype, int32_t b, const void* corpus,
                   const float* row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
                   const uint32_t* exclude, int64_t exclude_row_words, const uint32_t* masks,
                   int32_t nmasks, int64_t mask_words, const int64_t* ranges, int32_t nranges,
                   int32_t k, const float* out_scores, const int32_t* out_ids);
int topk_entry(const void* queries, int32_t query_dtype, int32_t b, const void* corpus,
               const float* row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
               const uint32_t* exclude, int64_t exclude_row_words, const uint32_t* masks,
               int32_t nmasks, int64_t mask_words, const int64_t* ranges, int32_t nranges,
               int32_t k, float* out_scores, int32_t* out_ids, void* workspace,
               size_t workspace_bytes, void* stream);
size_t workspace_bytes_for(int32_t b, int64_t n, int32_t d, int32_t k, int32_t qdt, int32_t cdt,
                           int32_t nmasks, int64_t candidates);

}  // namespace mips
