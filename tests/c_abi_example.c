/* The C ABI from plain C (no Python): build an f32 index, normalise a batch of queries,
 * search it with a shared exclusion bitmap, and check the result against a brute-force
 * scan of the same rows on the host (double precision, score descending then id
 * ascending, excluded ids skipped).
 * Exit status 0 on success; the first failure is printed. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mips.h"

#define N 5000
#define D 64
#define B 9
#define K 25

#define HIP_OK(x)                                                      \
  do {                                                                 \
    if ((x) != hipSuccess) {                                           \
      fprintf(stderr, "hip call failed at line %d\n", __LINE__);       \
      return 1;                                                        \
    }                                                                  \
  } while (0)
#define MIPS_OK_(x)                                                    \
  do {                                                                 \
    int rc_ = (x);                                                     \
    if (rc_ != MIPS_OK) {                                              \
      fprintf(stderr, "line %d: %s\n", __LINE__, mips_status_string(rc_)); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

static uint32_t lcg_state = 20261203u;
static float uniform(void) { /* in [-1, 1) */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)((lcg_state >> 8) & 0xFFFFFF) / 8388608.0f - 1.0f;
}

static void normalise(const float* x, double* y, int rows) {
  for (int r = 0; r < rows; ++r) {
    double s = 0.0;
    for (int j = 0; j < D; ++j) s += (double)x[r * D + j] * x[r * D + j];
    const double inv = 1.0 / sqrt(s > 1e-12 ? s : 1e-12);
    for (int j = 0; j < D; ++j) y[r * D + j] = x[r * D + j] * inv;
  }
}

int main(void) {
  static float x[N * D], q[B * D];
  static double xn[N * D], qn[B * D], sc[N];
  static uint32_t excl[(N + 31) / 32];
  static float out_s[B * K];
  static int32_t out_i[B * K];
  for (int i = 0; i < N * D; ++i) x[i] = uniform();
  for (int i = 0; i < B * D; ++i) q[i] = uniform();
  for (int i = 0; i < N; i += 7) excl[i >> 5] |= 1u << (i & 31); /* every 7th id excluded */

  float *dx, *dq, *dqn, *ds;
  void *dc, *dw;
  int32_t* di;
  uint32_t* dexcl;
  const int64_t cbytes = mips_corpus_bytes(N, D, MIPS_F32);
  const size_t wbytes = mips_topk_workspace_size(B, N, D, K, MIPS_F32, MIPS_F32);
  if (cbytes <= 0 || wbytes == 0) {
    fprintf(stderr, "size queries failed\n");
    return 1;
  }
  HIP_OK(hipMalloc((void**)&dx, sizeof x));
  HIP_OK(hipMalloc((void**)&dq, sizeof q));
  HIP_OK(hipMalloc((void**)&dqn, sizeof q));
  HIP_OK(hipMalloc(&dc, (size_t)cbytes));
  HIP_OK(hipMalloc(&dw, wbytes));
  HIP_OK(hipMalloc((void**)&ds, sizeof out_s));
  HIP_OK(hipMalloc((void**)&di, sizeof out_i));
  HIP_OK(hipMalloc((void**)&dexcl, sizeof excl));
  HIP_OK(hipMemcpy(dx, x, sizeof x, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dexcl, excl, sizeof excl, hipMemcpyHostToDevice));

  MIPS_OK_(mips_prepare_corpus(dx, N, 0, D, MIPS_F32, dc, NULL, NULL));
  MIPS_OK_(mips_l2_normalize(dq, B, D, MIPS_F32, dqn, NULL));
  MIPS_OK_(mips_topk(dqn, MIPS_F32, B, dc, NULL, MIPS_F32, N, D, dexcl, 0, K, ds, di, dw, wbytes,
                     NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(out_s, ds, sizeof out_s, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out_i, di, sizeof out_i, hipMemcpyDeviceToHost));

  normalise(x, xn, N);
  normalise(q, qn, B);
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i < N; ++i) {
      double s = 0.0;
      for (int j = 0; j < D; ++j) s += qn[b * D + j] * xn[i * D + j];
      sc[i] = s;
    }
    /* the exact K-th best score, by repeated selection (N is small) */
    static unsigned char taken[N];
    memset(taken, 0, sizeof taken);
    double kth = 0.0;
    for (int r = 0; r < K; ++r) {
      int best = -1;
      for (int i = 0; i < N; ++i) {
        if (taken[i] || (excl[i >> 5] >> (i & 31)) & 1u) continue;
        if (best < 0 || sc[i] > sc[best]) best = i;
      }
      taken[best] = 1;
      kth = sc[best];
    }
    for (int r = 0; r < K; ++r) {
      const int32_t id = out_i[b * K + r];
      const float s = out_s[b * K + r];
      if (id < 0 || id >= N || ((excl[id >> 5] >> (id & 31)) & 1u)) {
        fprintf(stderr, "query %d rank %d: bad id %d\n", b, r, id);
        return 1;
      }
      if (fabs((double)s - sc[id]) > 1e-5) {
        fprintf(stderr, "query %d rank %d: score %g, exact %g\n", b, r, s, sc[id]);
        return 1;
      }
      if (!taken[id] && fabs(sc[id] - kth) > 1e-5) {
        fprintf(stderr, "query %d rank %d: id %d is not in the exact top-%d\n", b, r, id, K);
        return 1;
      }
      if (r > 0) {
        const float p = out_s[b * K + r - 1];
        if (p < s || (p == s && out_i[b * K + r - 1] > id)) {
          fprintf(stderr, "query %d rank %d: out of order\n", b, r);
          return 1;
        }
      }
    }
  }
  hipFree(dx);
  hipFree(dq);
  hipFree(dqn);
  hipFree(dc);
  hipFree(dw);
  hipFree(ds);
  hipFree(di);
  hipFree(dexcl);
  printf("c abi ok: n=%d d=%d b=%d k=%d\n", N, D, B, K);
  return 0;
}
