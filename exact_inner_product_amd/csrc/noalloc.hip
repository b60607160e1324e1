// noalloc.hip -- mips_topk_noalloc: mips_topk with its scratch in a library-held device
// array instead of a caller-given workspace, for callers that cannot allocate.
//
// The array is a file-scope __device__ variable of this code object, so each device holds
// its own copy (MIPS_NOALLOC_SCRATCH_BYTES) from the first call on that device until the
// process ends. Host code never uses the array's name as an address: the device address
// comes from hipGetSymbolAddress, taken once per device with that device current.
#include <mutex>

#include "host.h"

namespace mips {

static __device__ __attribute__((aligned(256))) uint8_t scratch[MIPS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of the current device's scratch array; MIPS_OK or an error status.
static int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_last_hip_error(e);
    return MIPS_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return MIPS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_last_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return MIPS_ERR_HIP;
    }
    addr[dev] = p;
  }
  *out = addr[dev];
  return MIPS_OK;
}

}  // namespace mips

extern "C" {

int mips_topk_noalloc(const void* queries, int32_t query_dtype, int32_t b, const void* corpus,
                      const float* row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
                      const uint32_t* exclude, int64_t exclude_row_words, int32_t k,
                      float* out_scores, int32_t* out_ids, void* stream) {
  const int64_t whole[2] = {0, n};
  int rc = mips::validate_entry(queries, query_dtype, b, corpus, row_scale, corpus_dtype, n, d,
                                exclude, exclude_row_words, nullptr, 0, 0, whole, 1, k,
                                out_scores, out_ids);
  if (rc != MIPS_OK) return rc;
  // the call must fit with mips_topk's default candidate capacity
  const size_t need = mips::workspace_bytes_for(b, n, d, k, query_dtype, corpus_dtype, 0, -1);
  if (need == 0) return MIPS_ERR_UNSUPPORTED;
  if (need > MIPS_NOALLOC_SCRATCH_BYTES) return MIPS_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((rc = mips::scratch_address(&ws)) != MIPS_OK) return rc;
  // every flag, counter and list the passes read is written by an earlier pass of the same
  // call, so nothing in the scratch needs clearing
  return mips::topk_entry(queries, query_dtype, b, corpus, row_scale, corpus_dtype, n, d,
                          exclude, exclude_row_words, nullptr, 0, 0, whole, 1, k, out_scores,
                          out_ids, ws, MIPS_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
