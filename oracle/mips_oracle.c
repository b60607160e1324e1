/*
 * mips_oracle.c -- CPU oracle for exhaustive inner-product top-K.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * reference that the HIP library is checked against. Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it. It shares no code
 * with the HIP library and includes none of its headers.
 *
 * What it computes, and where the pages define it:
 *
 *  - l2 normalisation: y = x / sqrt(max(sum x^2, 1e-12)), the form of
 *    `_l2_normalize_candidates` and of the user-representation normalisation in
 *    recsys_two_tower_model.py (x-algorithm Phoenix). oracle_l2_normalize gives the
 *    value in fp64. The index build decides its stored codes from the row normalised
 *    in binary32, the precision of the Model's float32 tensors: the sum of squares in
 *    dimension order, the square root and each quotient rounded to binary32.
 *  - packing of the normalised index into a narrow type, as "normalise once at
 *    index time; store f16/int8" ("Two-tower retrieval", mhtirogla.ai, section
 *    "Implementation notes") and the bf16 `post_embeddings` index of
 *    recsys_two_tower_model.py. bf16 and OCP E4M3 codes are produced by
 *    round-to-nearest-even onto the format's value grid, derived here from the
 *    format definitions; E4M3 saturates at +-448 and uses one per-row scale,
 *    the smallest power of two 2^t with max|y| <= 448 * 2^t (a zero row gets 1).
 *  - int8 packing with one scale per row, the rule of the quantised scoring branch
 *    of `RecsysTwoTowerModel.forward` (its per-user quantisation, which the pages
 *    show; the index side is taken to follow the same rule): scale =
 *    max(max|y| / 127, 1e-12) as a float, code = y / scale rounded to nearest
 *    (ties to even) and clipped to [-127, 127]. The stored value is code * scale.
 *  - scoring: every query against every non-excluded corpus row by dot product
 *    (`RecsysTwoTowerModel.forward`: matmul of the users against the whole index,
 *    masked by one shared type mask; Phoenix README, "How Retrieval Works", step 4).
 *    Operands are decoded exactly to fp64 and summed in dimension order. Each
 *    product of two stored operands is exact in fp64, so the sums are exact up to
 *    the final fp64 roundings.
 *  - selection: a full sort of all eligible (score, id) pairs, by score descending
 *    and then id ascending (the stable full sort of the toy's `top_k` in
 *    "Two-tower retrieval", section "Code"), then the first min(k, eligible)
 *    entries (`local_top_k` takes min(k, N)). Missing entries are padded with
 *    (-inf, -1). Excluded ids are never returned.
 *
 *  - quantised scoring (oracle_topk_int8, oracle_scores_int8), the int8 branch of
 *    `RecsysTwoTowerModel.forward` (`compute_top_k_int8`) step by step, every step in
 *    binary32 as the Model's float32 tensors: per user, us = max(max_d |u_d| / 127,
 *    1e-12); uq_d = u_d / us rounded to nearest (ties to even) and clipped to
 *    [-127, 127]; the exact integer dot product acc of uq with the item's int8 codes;
 *    then acc times us, then times the item's scale. The page casts the product to
 *    bf16; here it stays binary32 (the scores are fp32 throughout this library).
 *  - quantisation of rows as given, without normalisation (oracle_quantize): the int8
 *    rule above, or E4M3 codes with the power-of-two scale of the index build (the
 *    reading used for the queries of an fp8 index).
 *
 *  - merging: the per-query union of several sorted (score, id) lists -- the
 *    results of separate indexes, each id shifted by its index's offset -- cut to
 *    the best k by the same order ("Two-Tower Retrieval at Industrial Scale",
 *    engineeringmaxxing.com: the fresh shard searched beside the base index and
 *    the two result lists merged by score). Padding entries (id -1) are skipped.
 *
 * Non-finite inputs are not supported; the entry points reject them.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2, OR_I8 = 3 };
enum { OR_OK = 0, OR_BAD_ARG = 1, OR_NONFINITE = 2, OR_NOMEM = 3 };

/* ------------------------------------------------------------------ formats */

/* bf16 is the upper 16 bits of an IEEE binary32. */
double oracle_bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal: m * 2^-9. Exponent 15 with mantissa 7 is NaN.
 * There are no infinities; the largest finite magnitude is 1.75 * 2^8 = 448. */
double oracle_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round |a| to the nearest multiple of `q` (a power of two), ties to even.
 * a / q is exact because q is a power of two; nearbyint uses the default
 * round-to-nearest-even mode. */
static double round_to_grid(double a, double q)
{
    return nearbyint(a / q) * q;
}

/* bf16 code of y by round-to-nearest-even. bf16 keeps 8 significant bits, so in
 * the binade [2^e, 2^(e+1)) the spacing is 2^(e-7); below the smallest normal
 * 2^-126 the spacing stays 2^-133. The sign is kept, also for zero. */
uint16_t oracle_bf16_from_f64(double y)
{
    uint16_t sign = signbit(y) ? 0x8000u : 0u;
    double a = fabs(y);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1; /* floor(log2 a) */
    if (ex < -126)
        ex = -126;
    double r = round_to_grid(a, ldexp(1.0, ex - 7));
    float f = (float)r; /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* Decoded values of all 256 E4M3 codes, filled once from oracle_e4m3_value. */
static double g_e4m3[256];
__attribute__((constructor)) static void fill_e4m3_table(void)
{
    for (int c = 0; c < 256; ++c)
        g_e4m3[c] = oracle_e4m3_value((uint8_t)c);
}

/* E4M3 code of v by round-to-nearest-even with saturation at 448. 4 significant
 * bits: spacing 2^(e-3) in the binade [2^e, 2^(e+1)); below the smallest normal
 * 2^-6 the spacing stays 2^-9. The code is found by matching the decoded grid: the
 * positive codes 0x00..0x7E decode in increasing order, so a binary search finds it. */
uint8_t oracle_e4m3_from_f64(double v)
{
    uint8_t sign = signbit(v) ? 0x80u : 0u;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1;
    if (ex < -6)
        ex = -6;
    double r = round_to_grid(a, ldexp(1.0, ex - 3));
    if (r > 448.0)
        r = 448.0;
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        int mid = (lo + hi) / 2;
        if (g_e4m3[mid] < r)
            lo = mid + 1;
        else
            hi = mid;
    }
    if (g_e4m3[lo] == r)
        return (uint8_t)(sign | lo);
    return 0xFF; /* unreachable for finite v */
}

/* Per-row E4M3 scale: the smallest power of two s = 2^t with amax <= 448 * s.
 * With amax = f * 2^e, f in [0.5, 1): amax <= 0.875 * 2^(9+t) holds for
 * t >= e - 9 when f <= 0.875, else for t >= e - 8. A zero row gets s = 1. */
double oracle_e4m3_row_scale(double amax)
{
    if (amax == 0.0)
        return 1.0;
    int e;
    double f = frexp(amax, &e);
    int t = (f <= 0.875) ? e - 9 : e - 8;
    return ldexp(1.0, t);
}

/* int8 per-row scale: the largest magnitude over 127, at least 1e-12, rounded to a
 * float (the scale is stored as a float). */
double oracle_i8_row_scale(double amax)
{
    return (double)(float)fmax(amax / 127.0, 1e-12);
}

/* int8 code of v: nearest integer, ties to even (nearbyint in the default rounding
 * mode), clipped to [-127, 127]. */
int8_t oracle_i8_from_f64(double v)
{
    double r = nearbyint(v);
    if (r > 127.0)
        r = 127.0;
    if (r < -127.0)
        r = -127.0;
    return (int8_t)r;
}

/* ------------------------------------------------------------ normalisation */

/* y[r, :] = x[r, :] / sqrt(max(sum_d x[r, d]^2, 1e-12)), all in fp64. */
int oracle_l2_normalize(const float *x, int64_t rows, int32_t d, double *y)
{
    if (!x || !y || rows < 0 || d <= 0)
        return OR_BAD_ARG;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * (int64_t)d;
        double ss = 0.0;
        for (int32_t j = 0; j < d; ++j) {
            if (!isfinite(xr[j]))
                return OR_NONFINITE;
            ss += (double)xr[j] * (double)xr[j];
        }
        double nrm = sqrt(fmax(ss, 1e-12));
        for (int32_t j = 0; j < d; ++j)
            y[r * (int64_t)d + j] = (double)xr[j] / nrm;
    }
    return OR_OK;
}

/* One row normalised in binary32: ss = sum of x_d * x_d in dimension order, nrm =
 * sqrt(max(ss, 1e-12)), y_d = x_d / nrm, every operation rounded to binary32 (the
 * build turns floating-point contraction off, so a product is rounded before its sum). */
static int normalize_row_f32(const float *xr, int32_t d, float *y)
{
    float ss = 0.0f;
    for (int32_t j = 0; j < d; ++j) {
        if (!isfinite(xr[j]))
            return OR_NONFINITE;
        ss = ss + xr[j] * xr[j];
    }
    const float nrm = sqrtf(fmaxf(ss, 1e-12f));
    for (int32_t j = 0; j < d; ++j)
        y[j] = xr[j] / nrm;
    return OR_OK;
}

/* Normalise `rows` raw rows (binary32, normalize_row_f32) and pack them row-major into
 * `out`; every code is decided from the binary32 value:
 *   OR_F32:  float  [rows, d]  (y itself)
 *   OR_BF16: uint16 [rows, d]  (bf16 codes)
 *   OR_E4M3: uint8  [rows, d]  (E4M3 codes of y / scale) and scale[rows] (float)
 *   OR_I8:   int8   [rows, d]  (int8 codes of y / scale, the quotient and the scale
 *            max(max|y| / 127, 1e-12) in binary32) and scale[rows] (float)
 */
int oracle_prepare(const float *x, int64_t rows, int32_t d, int32_t dtype, void *out,
                   float *scale)
{
    if (!x || !out || rows < 0 || d <= 0 || dtype < OR_F32 || dtype > OR_I8)
        return OR_BAD_ARG;
    if ((dtype == OR_E4M3 || dtype == OR_I8) && !scale)
        return OR_BAD_ARG;
    float *y = (float *)malloc(sizeof(float) * (size_t)d);
    if (!y)
        return OR_NOMEM;
    for (int64_t r = 0; r < rows; ++r) {
        int rc = normalize_row_f32(x + r * (int64_t)d, d, y);
        if (rc != OR_OK) {
            free(y);
            return rc;
        }
        int64_t base = r * (int64_t)d;
        float amax = 0.0f;
        for (int32_t j = 0; j < d; ++j)
            amax = fmaxf(amax, fabsf(y[j]));
        if (dtype == OR_F32) {
            for (int32_t j = 0; j < d; ++j)
                ((float *)out)[base + j] = y[j];
        } else if (dtype == OR_BF16) {
            for (int32_t j = 0; j < d; ++j)
                ((uint16_t *)out)[base + j] = oracle_bf16_from_f64((double)y[j]);
        } else if (dtype == OR_E4M3) {
            /* a power of two: y / s is exact */
            double s = oracle_e4m3_row_scale((double)amax);
            scale[r] = (float)s;
            for (int32_t j = 0; j < d; ++j)
                ((uint8_t *)out)[base + j] = oracle_e4m3_from_f64((double)y[j] / s);
        } else {
            const float s = fmaxf(amax / 127.0f, 1e-12f);
            scale[r] = s;
            for (int32_t j = 0; j < d; ++j)
                ((int8_t *)out)[base + j] = oracle_i8_from_f64((double)(y[j] / s));
        }
    }
    free(y);
    return OR_OK;
}

/* ---------------------------------------------------------------- scoring */

static double stored_value(int32_t dtype, const void *base, int64_t idx)
{
    switch (dtype) {
    case OR_F32:
        return (double)((const float *)base)[idx];
    case OR_BF16:
        return oracle_bf16_value(((const uint16_t *)base)[idx]);
    case OR_E4M3:
        return g_e4m3[((const uint8_t *)base)[idx]];
    default:
        return (double)((const int8_t *)base)[idx];
    }
}

/* Exact-as-fp64 score of query row `qrow` against corpus row `i`: the sum over
 * dimensions, in order, of q[j] * (stored value * row scale). (One loop per format, the
 * same arithmetic as stored_value element by element.) */
static double score_one(const double *q, int32_t c_dtype, const void *corpus,
                        const float *row_scale, int64_t i, int32_t d)
{
    double s = 0.0;
    double rs = (c_dtype == OR_E4M3 || c_dtype == OR_I8) ? (double)row_scale[i] : 1.0;
    const int64_t base = i * (int64_t)d;
    switch (c_dtype) {
    case OR_F32: {
        const float *c = (const float *)corpus + base;
        for (int32_t j = 0; j < d; ++j)
            s += q[j] * ((double)c[j] * rs);
        break;
    }
    case OR_BF16: {
        const uint16_t *c = (const uint16_t *)corpus + base;
        for (int32_t j = 0; j < d; ++j)
            s += q[j] * (oracle_bf16_value(c[j]) * rs);
        break;
    }
    case OR_E4M3: {
        const uint8_t *c = (const uint8_t *)corpus + base;
        for (int32_t j = 0; j < d; ++j)
            s += q[j] * (g_e4m3[c[j]] * rs);
        break;
    }
    default: {
        const int8_t *c = (const int8_t *)corpus + base;
        for (int32_t j = 0; j < d; ++j)
            s += q[j] * ((double)c[j] * rs);
        break;
    }
    }
    return s;
}

/* ------------------------------------------------------- quantised scoring */

/* The per-user int8 quantisation of the quantised scoring branch, in binary32: the
 * scale us = max(max_d |u_d| / 127, 1e-12) and the codes uq_d = u_d / us rounded to
 * nearest, ties to even, clipped to [-127, 127]. u is the row as given (f32 values). */
static float quantize_row_i8(const float *u, int32_t d, int32_t *uq)
{
    float amax = 0.0f;
    for (int32_t j = 0; j < d; ++j)
        amax = fmaxf(amax, fabsf(u[j]));
    const float us = fmaxf(amax / 127.0f, 1e-12f);
    for (int32_t j = 0; j < d; ++j) {
        const float t = u[j] / us; /* one binary32 division */
        uq[j] = (int32_t)oracle_i8_from_f64((double)t);
    }
    return us;
}

/* Score of one item in the quantised branch: the exact integer dot product of the user's
 * codes with the item's codes, then times the user scale, then times the item scale,
 * each product rounded to binary32. */
static float score_int8_row(const int32_t *uq, float us, const int8_t *codes, float scale,
                            int32_t d)
{
    int64_t acc = 0;
    for (int32_t j = 0; j < d; ++j)
        acc += (int64_t)uq[j] * (int64_t)codes[j];
    const float a = (float)acc; /* |acc| <= 127 * 127 * d < 2^24: exact */
    const float t = a * us;
    return t * scale;
}

/* The f32 value of element idx of a query buffer (OR_F32 or OR_BF16); exact. */
static float query_f32(int32_t dtype, const void *base, int64_t idx)
{
    return (float)stored_value(dtype, base, idx);
}

/* Rows as given (OR_F32 or OR_BF16 values, [rows, d]) quantised without normalisation:
 *   OR_I8:   codes int8 [rows, d] and scale[rows], the per-user rule of the quantised
 *            branch (quantize_row_i8);
 *   OR_E4M3: codes uint8 [rows, d], E4M3 of x / s with s the smallest power of two with
 *            max|x| <= 448 s (1 for a zero row), and scale[rows] = s. */
int oracle_quantize(int32_t x_dtype, const void *x, int64_t rows, int32_t d, int32_t dtype,
                    void *codes, float *scale)
{
    if (!x || !codes || !scale || rows < 0 || d <= 0)
        return OR_BAD_ARG;
    if ((x_dtype != OR_F32 && x_dtype != OR_BF16) || (dtype != OR_I8 && dtype != OR_E4M3))
        return OR_BAD_ARG;
    float *u = (float *)malloc(sizeof(float) * (size_t)d);
    int32_t *uq = (int32_t *)malloc(sizeof(int32_t) * (size_t)d);
    if (!u || !uq) {
        free(u);
        free(uq);
        return OR_NOMEM;
    }
    int rc = OR_OK;
    for (int64_t r = 0; r < rows && rc == OR_OK; ++r) {
        for (int32_t j = 0; j < d; ++j) {
            u[j] = query_f32(x_dtype, x, r * (int64_t)d + j);
            if (!isfinite(u[j]))
                rc = OR_NONFINITE;
        }
        if (rc != OR_OK)
            break;
        if (dtype == OR_I8) {
            scale[r] = quantize_row_i8(u, d, uq);
            for (int32_t j = 0; j < d; ++j)
                ((int8_t *)codes)[r * (int64_t)d + j] = (int8_t)uq[j];
        } else {
            float amax = 0.0f;
            for (int32_t j = 0; j < d; ++j)
                amax = fmaxf(amax, fabsf(u[j]));
            const double s = oracle_e4m3_row_scale((double)amax);
            scale[r] = (float)s;
            for (int32_t j = 0; j < d; ++j)
                ((uint8_t *)codes)[r * (int64_t)d + j] = oracle_e4m3_from_f64((double)u[j] / s);
        }
    }
    free(u);
    free(uq);
    return rc;
}

static int excluded(const uint32_t *bits, int64_t i)
{
    return bits && ((bits[i >> 5] >> (i & 31)) & 1u);
}

typedef struct {
    double s;
    int32_t id;
} pair_t;

/* Score descending, then id ascending. */
static int cmp_pair(const void *a, const void *b)
{
    const pair_t *x = (const pair_t *)a, *y = (const pair_t *)b;
    if (x->s > y->s)
        return -1;
    if (x->s < y->s)
        return 1;
    return (x->id > y->id) - (x->id < y->id);
}

typedef struct {
    int32_t q_dtype, c_dtype, d, k, b, m; /* m query rows per result row (interests) */
    int quantised; /* int8 index scored by the quantised branch (score_int8_row) */
    const void *queries, *corpus;
    const float *row_scale;
    const uint32_t *exclude;
    int64_t n;
    double *out_s;
    int32_t *out_id;
    int next; /* next query to take (guarded by lock) */
    int status;
    pthread_mutex_t lock;
} topk_job_t;

static void *topk_worker(void *arg)
{
    topk_job_t *J = (topk_job_t *)arg;
    pair_t *pairs = (pair_t *)malloc(sizeof(pair_t) * (size_t)(J->n > 0 ? J->n : 1));
    double *q = (double *)malloc(sizeof(double) * (size_t)J->d * (size_t)J->m);
    float *qf = (float *)malloc(sizeof(float) * (size_t)J->d);
    int32_t *uq = (int32_t *)malloc(sizeof(int32_t) * (size_t)J->d * (size_t)J->m);
    float *usv = (float *)malloc(sizeof(float) * (size_t)J->m);
    if (!pairs || !q || !qf || !uq || !usv) {
        pthread_mutex_lock(&J->lock);
        J->status = OR_NOMEM;
        pthread_mutex_unlock(&J->lock);
        free(pairs);
        free(q);
        free(qf);
        free(uq);
        free(usv);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int b = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (b >= J->b)
            break;
        /* result row b: query rows b*m .. b*m+m-1; an item scores its best match */
        for (int64_t j = 0; j < (int64_t)J->d * J->m; ++j)
            q[j] = stored_value(J->q_dtype, J->queries, (int64_t)b * J->m * J->d + j);
        if (J->quantised)
            for (int32_t v = 0; v < J->m; ++v) {
                for (int32_t j = 0; j < J->d; ++j)
                    qf[j] = (float)q[(int64_t)v * J->d + j];
                usv[v] = quantize_row_i8(qf, J->d, uq + (int64_t)v * J->d);
            }
        int64_t m = 0;
        for (int64_t i = 0; i < J->n; ++i) {
            if (excluded(J->exclude, i))
                continue;
            if (J->quantised) {
                const int8_t *row = (const int8_t *)J->corpus + i * (int64_t)J->d;
                float best = score_int8_row(uq, usv[0], row, J->row_scale[i], J->d);
                for (int32_t v = 1; v < J->m; ++v) {
                    const float sv = score_int8_row(uq + (int64_t)v * J->d, usv[v], row,
                                                    J->row_scale[i], J->d);
                    if (sv > best)
                        best = sv;
                }
                pairs[m].s = (double)best;
                pairs[m].id = (int32_t)i;
                ++m;
                continue;
            }
            double best = score_one(q, J->c_dtype, J->corpus, J->row_scale, i, J->d);
            for (int32_t v = 1; v < J->m; ++v) {
                double sv = score_one(q + (int64_t)v * J->d, J->c_dtype, J->corpus,
                                      J->row_scale, i, J->d);
                if (sv > best)
                    best = sv;
            }
            pairs[m].s = best;
            pairs[m].id = (int32_t)i;
            ++m;
        }
        qsort(pairs, (size_t)m, sizeof(pair_t), cmp_pair);
        for (int32_t t = 0; t < J->k; ++t) {
            int64_t o = (int64_t)b * J->k + t;
            if (t < m) {
                J->out_s[o] = pairs[t].s;
                J->out_id[o] = pairs[t].id;
            } else {
                J->out_s[o] = -INFINITY;
                J->out_id[o] = -1;
            }
        }
    }
    free(pairs);
    free(q);
    free(qf);
    free(uq);
    free(usv);
    return NULL;
}

static int check_finite(int32_t dtype, const void *p, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        if (!isfinite(stored_value(dtype, p, i)))
            return 0;
    return 1;
}

/* Top-k of every query against the whole corpus.
 *   queries:  [b, d] row-major, q_dtype OR_F32 or OR_BF16
 *   corpus:   [n, d] row-major, c_dtype OR_F32, OR_BF16, OR_E4M3 or OR_I8
 *   row_scale:[n] for OR_E4M3 and OR_I8, else ignored
 *   exclude:  NULL or uint32[ceil(n/32)], bit (i & 31) of word (i >> 5) excludes id i
 *   out_s:    [b, k] fp64 scores, out_id: [b, k] int32 ids
 */
static int topk_m(int32_t q_dtype, const void *queries, int32_t b, int32_t mq, int32_t c_dtype,
                  const void *corpus, const float *row_scale, int64_t n, int32_t d,
                  const uint32_t *exclude, int32_t k, double *out_s, int32_t *out_id,
                  int32_t threads, int quantised);

int oracle_topk(int32_t q_dtype, const void *queries, int32_t b, int32_t c_dtype,
                const void *corpus, const float *row_scale, int64_t n, int32_t d,
                const uint32_t *exclude, int32_t k, double *out_s, int32_t *out_id,
                int32_t threads)
{
    return topk_m(q_dtype, queries, b, 1, c_dtype, corpus, row_scale, n, d, exclude, k, out_s,
                  out_id, threads, 0);
}

/* Top-k of every query against an int8 index by the quantised branch of
 * `RecsysTwoTowerModel.forward` (quantize_row_i8, score_int8_row): each query quantised
 * to int8 with its own scale, exact integer dot products, then the user scale and the
 * item scale in binary32. Arguments as oracle_topk with c_dtype OR_I8; out_s holds the
 * binary32 scores (exactly, as doubles). */
int oracle_topk_int8(int32_t q_dtype, const void *queries, int32_t b, const void *corpus,
                     const float *row_scale, int64_t n, int32_t d, const uint32_t *exclude,
                     int32_t k, double *out_s, int32_t *out_id, int32_t threads)
{
    return topk_m(q_dtype, queries, b, 1, OR_I8, corpus, row_scale, n, d, exclude, k, out_s,
                  out_id, threads, 1);
}

/* Top-k of b users with m query vectors each (queries [b * m, d], user-major): an item's
 * score is its best dot product over the user's vectors (the max over interest vectors
 * of "Two-Tower Retrieval at Industrial Scale", section "Beyond Dot Products"). */
int oracle_maxsim_topk(int32_t q_dtype, const void *queries, int32_t b, int32_t m,
                       int32_t c_dtype, const void *corpus, const float *row_scale, int64_t n,
                       int32_t d, const uint32_t *exclude, int32_t k, double *out_s,
                       int32_t *out_id, int32_t threads)
{
    if (m < 1)
        return OR_BAD_ARG;
    return topk_m(q_dtype, queries, b, m, c_dtype, corpus, row_scale, n, d, exclude, k, out_s,
                  out_id, threads, 0);
}

/* As oracle_maxsim_topk against an int8 index, each vector scored by the quantised
 * branch (as oracle_topk_int8); an item scores its best over the user's vectors. */
int oracle_maxsim_topk_int8(int32_t q_dtype, const void *queries, int32_t b, int32_t m,
                            const void *corpus, const float *row_scale, int64_t n, int32_t d,
                            const uint32_t *exclude, int32_t k, double *out_s, int32_t *out_id,
                            int32_t threads)
{
    if (m < 1)
        return OR_BAD_ARG;
    return topk_m(q_dtype, queries, b, m, OR_I8, corpus, row_scale, n, d, exclude, k, out_s,
                  out_id, threads, 1);
}

static int topk_m(int32_t q_dtype, const void *queries, int32_t b, int32_t mq, int32_t c_dtype,
                  const void *corpus, const float *row_scale, int64_t n, int32_t d,
                  const uint32_t *exclude, int32_t k, double *out_s, int32_t *out_id,
                  int32_t threads, int quantised)
{
    if (!queries || !corpus || !out_s || !out_id || b < 0 || n < 0 || d <= 0 || k <= 0)
        return OR_BAD_ARG;
    if (q_dtype != OR_F32 && q_dtype != OR_BF16)
        return OR_BAD_ARG;
    if (c_dtype < OR_F32 || c_dtype > OR_I8 ||
        ((c_dtype == OR_E4M3 || c_dtype == OR_I8) && !row_scale))
        return OR_BAD_ARG;
    if (!check_finite(q_dtype, queries, (int64_t)b * mq * d) ||
        !check_finite(c_dtype, corpus, n * (int64_t)d))
        return OR_NONFINITE;
    if (c_dtype == OR_E4M3 || c_dtype == OR_I8)
        for (int64_t i = 0; i < n; ++i)
            if (!isfinite(row_scale[i]))
                return OR_NONFINITE;

    topk_job_t J;
    memset(&J, 0, sizeof J);
    J.q_dtype = q_dtype;
    J.c_dtype = c_dtype;
    J.d = d;
    J.k = k;
    J.b = b;
    J.m = mq;
    J.quantised = quantised;
    J.queries = queries;
    J.corpus = corpus;
    J.row_scale = row_scale;
    J.exclude = exclude;
    J.n = n;
    J.out_s = out_s;
    J.out_id = out_id;
    pthread_mutex_init(&J.lock, NULL);
    if (threads < 1)
        threads = 1;
    if (threads > b && b > 0)
        threads = b;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)threads);
    int started = 0;
    for (int t = 0; t < threads; ++t)
        if (pthread_create(&tid[t], NULL, topk_worker, &J) == 0)
            ++started;
    if (started == 0)
        topk_worker(&J);
    for (int t = 0; t < started; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    pthread_mutex_destroy(&J.lock);
    return J.status;
}

/* Exact scores of given (query, id) pairs: out[t] = score(queries[qidx[t]], corpus[ids[t]]). */
int oracle_scores(int32_t q_dtype, const void *queries, int32_t b, int32_t c_dtype,
                  const void *corpus, const float *row_scale, int64_t n, int32_t d,
                  const int32_t *qidx, const int32_t *ids, int64_t count, double *out)
{
    if (!queries || !corpus || !qidx || !ids || !out || d <= 0)
        return OR_BAD_ARG;
    double *q = (double *)malloc(sizeof(double) * (size_t)d);
    if (!q)
        return OR_NOMEM;
    for (int64_t t = 0; t < count; ++t) {
        if (qidx[t] < 0 || qidx[t] >= b || ids[t] < 0 || ids[t] >= n) {
            free(q);
            return OR_BAD_ARG;
        }
        for (int32_t j = 0; j < d; ++j)
            q[j] = stored_value(q_dtype, queries, (int64_t)qidx[t] * d + j);
        out[t] = score_one(q, c_dtype, corpus, row_scale, ids[t], d);
    }
    free(q);
    return OR_OK;
}

/* Quantised-branch scores of given (query, id) pairs against an int8 index:
 * out[t] = score_int8_row of query qidx[t] (quantised by quantize_row_i8) and row ids[t]. */
int oracle_scores_int8(int32_t q_dtype, const void *queries, int32_t b, const void *corpus,
                       const float *row_scale, int64_t n, int32_t d, const int32_t *qidx,
                       const int32_t *ids, int64_t count, double *out)
{
    if (!queries || !corpus || !row_scale || !qidx || !ids || !out || d <= 0 ||
        (q_dtype != OR_F32 && q_dtype != OR_BF16))
        return OR_BAD_ARG;
    float *u = (float *)malloc(sizeof(float) * (size_t)d);
    int32_t *uq = (int32_t *)malloc(sizeof(int32_t) * (size_t)d);
    if (!u || !uq) {
        free(u);
        free(uq);
        return OR_NOMEM;
    }
    int rc = OR_OK;
    for (int64_t t = 0; t < count; ++t) {
        if (qidx[t] < 0 || qidx[t] >= b || ids[t] < 0 || ids[t] >= n) {
            rc = OR_BAD_ARG;
            break;
        }
        for (int32_t j = 0; j < d; ++j)
            u[j] = query_f32(q_dtype, queries, (int64_t)qidx[t] * d + j);
        const float us = quantize_row_i8(u, d, uq);
        out[t] = (double)score_int8_row(uq, us, (const int8_t *)corpus + (int64_t)ids[t] * d,
                                        row_scale[ids[t]], d);
    }
    free(u);
    free(uq);
    return rc;
}

/* Merge of p sorted lists per query: in_s/in_id are [p, b, k_in] (list-major), a
 * list's ids are shifted by offsets[list]; entries with id < 0 are padding. The
 * result per query is the first k_out of all real entries sorted by score
 * descending, then id ascending, padded with (-inf, -1). */
int oracle_merge_topk(const float *in_s, const int32_t *in_id, const int64_t *offsets,
                      int32_t p, int32_t b, int32_t k_in, int32_t k_out, float *out_s,
                      int32_t *out_id)
{
    if (!in_s || !in_id || !offsets || !out_s || !out_id || p < 1 || b < 0 || k_in < 1 ||
        k_out < 1)
        return OR_BAD_ARG;
    pair_t *pairs = (pair_t *)malloc(sizeof(pair_t) * (size_t)p * (size_t)k_in);
    if (!pairs)
        return OR_NOMEM;
    for (int32_t q = 0; q < b; ++q) {
        int64_t m = 0;
        for (int32_t l = 0; l < p; ++l)
            for (int32_t j = 0; j < k_in; ++j) {
                int64_t o = ((int64_t)l * b + q) * k_in + j;
                if (in_id[o] < 0)
                    continue;
                if (!isfinite(in_s[o])) {
                    free(pairs);
                    return OR_NONFINITE;
                }
                pairs[m].s = (double)in_s[o];
                pairs[m].id = (int32_t)(in_id[o] + offsets[l]);
                ++m;
            }
        qsort(pairs, (size_t)m, sizeof(pair_t), cmp_pair);
        for (int32_t t = 0; t < k_out; ++t) {
            int64_t o = (int64_t)q * k_out + t;
            out_s[o] = t < m ? (float)pairs[t].s : -INFINITY;
            out_id[o] = t < m ? pairs[t].id : -1;
        }
    }
    free(pairs);
    return OR_OK;
}
