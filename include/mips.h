/*
 * mips.h -- C ABI of the MI355X (gfx950) exhaustive inner-product top-K library.
 *
 * The operation is the serving step of two-tower retrieval: a batch of L2-normalised
 * user embeddings queries[B, D] is scored by dot product against a precomputed,
 * L2-normalised candidate index corpus[N, D], and each user gets its K best candidates
 * (Phoenix README, "How Retrieval Works", steps 1-4; `RecsysTwoTowerModel.forward` in
 * recsys_two_tower_model.py, x-algorithm Phoenix, which scores the users against the
 * whole index, masks it with one shared type mask and takes a sorted top-min(k, N)).
 * The score matrix is never written to memory.
 *
 * Entry points: mips_l2_normalize and mips_prepare_corpus (normalisation, index build);
 * mips_topk (one result set per query), mips_topk_ranges (one per id range) and
 * mips_topk_masks (one per exclusion mask, from one pass over the index), with their
 * workspace sizes; mips_topk_noalloc (mips_topk with library-held scratch);
 * mips_merge_topk and mips_merge_interests (merges of sorted result lists);
 * mips_type_bitmap (per-type exclusion bitmaps); status strings and a timing hook.
 *
 * Conventions shared by every entry point:
 *  - All buffers are caller-owned (except the static scratch array of
 *    mips_topk_noalloc). Pointers marked "device" are HIP device memory; the library
 *    never allocates, frees or synchronises. Work is enqueued on
 *    `stream` (a hipStream_t; NULL is the default stream) and the call returns after
 *    enqueueing. Results are visible once the stream has reached that point.
 *  - Arguments are validated on the host before anything is enqueued. On any error
 *    nothing is enqueued and no output is touched. A failed launch returns
 *    MIPS_ERR_HIP; mips_last_hip_error() then gives the HIP error code (per thread).
 *    Faults inside kernels surface at the caller's next synchronisation.
 *  - Inputs must be finite. NaN and infinities are not supported.
 *  - Element types: MIPS_F32 (IEEE binary32), MIPS_BF16 (the upper 16 bits of a
 *    binary32), MIPS_FP8_E4M3 (OCP 8-bit float E4M3: bias 7, 3 mantissa bits, no
 *    infinities, max 448) and MIPS_INT8 (two's complement, -127..127), the last two
 *    always with one float scale per row.
 */
#ifndef MIPS_H
#define MIPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Entry points are the only symbols the shared library exports. */
#define MIPS_API __attribute__((visibility("default")))

#define MIPS_F32 0
#define MIPS_BF16 1
#define MIPS_FP8_E4M3 2
#define MIPS_INT8 3

#define MIPS_OK 0
#define MIPS_ERR_INVALID_ARG 1
#define MIPS_ERR_UNSUPPORTED 2
#define MIPS_ERR_WORKSPACE 3
#define MIPS_ERR_HIP 4

/* Largest supported K. */
#define MIPS_K_MAX 1024

/* Largest supported number of result lists per call: b for mips_topk, mips_topk_ranges and
 * the merges, b * nmasks for mips_topk_masks. Each list is one 256-thread workgroup of a
 * launch, whose work-item count must stay below 2^32. */
#define MIPS_B_MAX 8388608

/*
 * Packed corpus layout ("fragment-tiled"). Rows are grouped in blocks of 32
 * (N is padded up to a multiple of 32 with zero rows). Block g covers rows
 * 32g..32g+31 and occupies 32*D*E bytes (E = 4, 2 or 1 bytes per element), split into
 * 1 KiB chunks of 64 slots x 16 bytes. Slot s of chunk c holds row 32g + (s & 31) and
 * the following dimensions, with h = s >> 5 and t the element index inside the slot:
 *   MIPS_F32      (4 per slot):  dim = 8c + 2t + h
 *   MIPS_BF16     (8 per slot):  dim = 16c + 8h + t
 *   MIPS_FP8_E4M3 (16 per slot): dim = 64(c >> 1) + 32h + 16(c & 1) + t
 *   MIPS_INT8     (16 per slot): dim = 32c + 16h + t
 * Every 16-byte slot is exactly one lane's operand of the gfx950 32x32 MFMA, so the
 * score kernel streams the corpus from HBM with fully coalesced 1 KiB wave loads and
 * no LDS transpose. For MIPS_FP8_E4M3 and MIPS_INT8 the per-row scale array has one
 * float per padded row (see mips_prepare_corpus); fp8 scales are powers of two.
 */

/* Bytes of a packed corpus of n rows (n >= 1) and width d; -1 if unsupported. */
MIPS_API int64_t mips_corpus_bytes(int64_t n, int32_t d, int32_t dtype);

/* Number of floats in the per-row scale array of an n-row corpus (n rounded up to 32). */
MIPS_API int64_t mips_scale_count(int64_t n);

/*
 * mips_l2_normalize -- y = x / sqrt(max(sum_d x^2, 1e-12)) per row, the form of
 * `_l2_normalize_candidates` and of the user-representation normalisation in
 * recsys_two_tower_model.py. Computed in fp32; the bf16 output is rounded to nearest
 * even.
 *   src   device, float [rows, d] row-major, finite.
 *   rows  >= 0 (0 enqueues nothing); d in [1, 4096].
 *   out_dtype  MIPS_F32 or MIPS_BF16.
 *   dst   device, [rows, d] row-major of out_dtype; may not alias src.
 * Errors: INVALID_ARG for NULL pointers, rows < 0, d out of range, misaligned pointers
 * (4 bytes for float, 2 for bf16); UNSUPPORTED for another out_dtype.
 */
MIPS_API int mips_l2_normalize(const float *src, int64_t rows, int32_t d, int32_t out_dtype, void *dst,
                      void *stream);

/*
 * mips_prepare_corpus -- the offline index build: normalise raw rows as
 * mips_l2_normalize does and pack them into the fragment-tiled layout ("normalise once
 * at index time; store f16/int8", "Two-tower retrieval", mhtirogla.ai, section
 * "Implementation notes"; the bf16 `post_embeddings` index of recsys_two_tower_model.py).
 *   src         device, float [rows, d] row-major: logical rows
 *               row_offset .. row_offset+rows-1 of the corpus.
 *   row_offset  multiple of 32 (lets a large corpus be packed in chunks).
 *   rows        >= 1. If rows is not a multiple of 32, this must be the last chunk: the
 *               rest of the last block is written as zero rows (with a zero row's
 *               scale: 1 for fp8, 1e-12 for int8).
 *   d           16, 32, 64, 128 or 256 (MIPS_F32: up to 128; MIPS_FP8_E4M3: 64, 128,
 *               256; MIPS_INT8: 32 .. 256).
 *   dtype       MIPS_F32 (rounded to nearest), MIPS_BF16 (nearest even),
 *               MIPS_FP8_E4M3: per row, scale s = the smallest power of two with
 *               max|y| <= 448 s (1 for a zero row) and codes = E4M3(y / s), nearest even,
 *               saturating; or MIPS_INT8: per row, scale s = max(max|y| / 127, 1e-12)
 *               and codes = y / s rounded to nearest (ties to even), clipped to
 *               [-127, 127] -- the per-row rule of the quantised scoring branch of
 *               `RecsysTwoTowerModel.forward` (recsys_two_tower_model.py).
 *   dst         device, packed corpus of at least mips_corpus_bytes(row_offset + rows).
 *   row_scale   device float [mips_scale_count(row_offset + rows)] for MIPS_FP8_E4M3 and
 *               MIPS_INT8 (entries row_offset.. are written), NULL otherwise.
 * Errors: INVALID_ARG (NULL, rows < 1, row_offset < 0 or not a multiple of 32, dst not
 * 16-byte aligned, row_scale missing for fp8 or int8), UNSUPPORTED (d or dtype).
 */
MIPS_API int mips_prepare_corpus(const float *src, int64_t rows, int64_t row_offset, int32_t d,
                        int32_t dtype, void *dst, float *row_scale, void *stream);

/*
 * mips_topk_workspace_size -- bytes of device workspace mips_topk needs for these
 * sizes with its default candidate capacity (about max(16 k, 32768) per query, at most
 * the corpus). A larger workspace raises the per-query candidate capacity; see
 * mips_topk. Returns 0 for unsupported arguments. The size depends on the current
 * device's compute-unit count (the candidate lists are split into one segment per
 * corpus slice, at most one slice per compute unit).
 */
MIPS_API size_t mips_topk_workspace_size(int32_t b, int64_t n, int32_t d, int32_t k,
                                int32_t query_dtype, int32_t corpus_dtype);

/*
 * mips_topk_workspace_size_for -- as mips_topk_workspace_size, for a candidate capacity
 * of at least candidates_per_query (>= 1) per query instead of the default. A capacity
 * below the number of candidates a query produces makes mips_topk rescan that query
 * (slower, same result). Returns 0 for unsupported arguments.
 */
MIPS_API size_t mips_topk_workspace_size_for(int32_t b, int64_t n, int32_t d, int32_t k,
                                    int32_t query_dtype, int32_t corpus_dtype,
                                    int64_t candidates_per_query);

/*
 * mips_topk -- exact top-k by inner product of every query against every corpus row
 * that the exclusion bitmap does not mask ("already seen"), with ties broken by
 * score descending, then id ascending.
 *   queries      device, [b, d] row-major, query_dtype MIPS_F32 or MIPS_BF16, assumed
 *                L2-normalised (use mips_l2_normalize); 4-byte aligned.
 *   b            1 .. MIPS_B_MAX.
 *   corpus       device, packed by mips_prepare_corpus (n rows, width d, corpus_dtype);
 *                16-byte aligned.
 *   row_scale    device, per-row scales for MIPS_FP8_E4M3 and MIPS_INT8 (NULL
 *                otherwise).
 *   corpus_dtype with query_dtype: F32/F32, BF16 with F32 or BF16 queries (queries are
 *                rounded to bf16), FP8_E4M3 with F32 or BF16 queries (each query row is
 *                quantised to E4M3 with its own power-of-two scale, the rule of
 *                mips_prepare_corpus), INT8 with F32 or BF16 queries (each query row is
 *                quantised to int8 with its own scale max|q| / 127, as the quantised
 *                branch of `RecsysTwoTowerModel.forward` does; the int32 dot product of
 *                the codes is scaled by the row scale, then by the query scale).
 *   n            1 .. 2^31 - 64.  d: as mips_prepare_corpus.
 *   exclude      device or NULL: bit (i & 31) of word (i >> 5) set means id i is never
 *                returned. With exclude_row_words == 0, one uint32 [ceil(n/32)] bitmap
 *                serves the whole batch; with exclude_row_words = w > 0, query q's own
 *                bitmap starts at word q * w (uint32 [b, w], w >= ceil(n/32)): a
 *                per-user set, such as the engagement history that hard-negative
 *                mining removes from each user's retrieved top-k ("Two-Tower Retrieval
 *                at Industrial Scale", section "When hard is too hard"). The sampled thresholds ignore per-query bitmaps, so
 *                a query whose own bitmap removes many of its best rows is rescued (exact,
 *                slower).
 *   exclude_row_words  0 or >= ceil(n/32), as above; > 0 needs a non-NULL exclude.
 *   k            1 .. MIPS_K_MAX.
 *   out_scores   device float [b, k]; out_ids device int32 [b, k]. Row q holds query q's
 *                min(k, eligible) best (score, id) pairs, score descending then id
 *                ascending; remaining slots are (-INFINITY, -1). Scores are fp32
 *                accumulations of the stored operands (no temperature is applied).
 *   workspace    device, 256-byte aligned; the fixed part plus at least one candidate
 *                per query and list segment (mips_topk_workspace_size gives the default,
 *                mips_topk_workspace_size_for any other capacity); its contents are
 *                undefined between calls, except two diagnostic counts (uint32) that the
 *                call's last pass leaves in bytes 0..7: the result lists queued for the
 *                rescue pass, and the lists resolved by the exact one-workgroup rescan
 *                (slow; 0 unless a rescue pass also overflows). Calls that share a
 *                workspace must be ordered on one stream.
 * Errors: INVALID_ARG (NULL where a buffer is required, b/n/k out of range, fp8 or int8
 * without row_scale, misalignment), UNSUPPORTED (d, k > MIPS_K_MAX, b > MIPS_B_MAX, dtype
 * pair), WORKSPACE (workspace_bytes too small), HIP (a launch failed); INVALID_ARG also for
 * exclude_row_words < 0, or > 0 with a NULL exclude or below ceil(n/32).
 */
MIPS_API int mips_topk(const void *queries, int32_t query_dtype, int32_t b, const void *corpus,
              const float *row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
              const uint32_t *exclude, int64_t exclude_row_words, int32_t k,
              float *out_scores, int32_t *out_ids, void *workspace, size_t workspace_bytes,
              void *stream);

/*
 * mips_topk_noalloc -- mips_topk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * search, arguments, ordering, padding and errors, with no workspace argument. Its scratch
 * is a device array held by the library, MIPS_NOALLOC_SCRATCH_BYTES per device, from the
 * first call on a device until the process ends; the call allocates and frees nothing.
 * Every call on one device shares that device's array: calls that overlap on a device (on
 * different streams, or from several threads without ordering) race and give undefined
 * results. The array keeps the last call's contents; a call reads nothing it did not write.
 * Errors: as mips_topk; WORKSPACE when mips_topk_workspace_size for the same arguments
 * exceeds MIPS_NOALLOC_SCRATCH_BYTES (e.g. b = 256, n = 10^7, d = 128, k = 500 fits, about
 * 76 MB; b = 1024, n = 10^8 does not); HIP when the array's address cannot be had.
 */
#define MIPS_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
MIPS_API int mips_topk_noalloc(const void *queries, int32_t query_dtype, int32_t b,
                               const void *corpus, const float *row_scale, int32_t corpus_dtype,
                               int64_t n, int32_t d, const uint32_t *exclude,
                               int64_t exclude_row_words, int32_t k, float *out_scores,
                               int32_t *out_ids, void *stream);

/*
 * mips_topk_ranges -- mips_topk restricted to id ranges, one result set per range: for
 * range r = [ranges[2r], ranges[2r+1]), the exact top-k of the non-excluded rows with ids
 * in the range (the dataset_ranges path of `RecsysTwoTowerModel.forward` in
 * recsys_two_tower_model.py, which slices the scores to [start, end), takes a sorted
 * top-k and adds start to the indices). Each range's pass reads only the blocks that hold
 * its rows, so disjoint ranges read the corpus once in all.
 *   ranges       host int64 [nranges][2]: 0 <= start < end <= n; ranges may overlap.
 *   nranges      >= 1.
 *   out_scores   device float [nranges, b, k]; out_ids device int32 [nranges, b, k]:
 *                range r's result, as mips_topk's, with absolute ids.
 *   The other arguments, the ordering, the padding and the workspace are as mips_topk's
 *   (the workspace for the whole corpus serves every range; ranges run one after the
 *   other on the stream).
 * Errors: as mips_topk, plus INVALID_ARG for a NULL ranges, nranges < 1 or a range outside
 * [0, n) or empty.
 */
MIPS_API int mips_topk_ranges(const void *queries, int32_t query_dtype, int32_t b, const void *corpus,
                              const float *row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
                              const uint32_t *exclude, int64_t exclude_row_words,
                              const int64_t *ranges, int32_t nranges,
                              int32_t k, float *out_scores, int32_t *out_ids, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * mips_topk_masks -- several result sets from one pass over the corpus: for each of the
 * nmasks exclusion masks, every query's exact top-k of the rows that mask does not
 * exclude. This is the per-type loop of `RecsysTwoTowerModel.forward`
 * (recsys_two_tower_model.py), which scores the batch once and takes one masked top-k per
 * target type; here each score is computed once and tested against the threshold of each
 * mask that admits its row. Masks may overlap.
 *   masks        device uint32 [nmasks][mask_words]: bit (i & 31) of word (i >> 5) of row t
 *                set means id i is not in result set t (mips_type_bitmap builds one per
 *                item type, with a shared exclusion folded in).
 *   nmasks       1 .. MIPS_MAX_MASKS.  mask_words >= ceil(n/32).
 *   out_scores   device float [nmasks, b, k]; out_ids device int32 [nmasks, b, k]: result
 *                set t of query q at [t][q], as mips_topk's row q.
 *   workspace    mips_topk_masks_workspace_size bytes: the fixed part and candidate lists
 *                per mask and query, of candidates_per_list entries each (< 1: the default
 *                capacity, as mips_topk_workspace_size; 0 returned for invalid sizes).
 *   The other arguments, the ordering and the padding are as mips_topk's.
 * Errors: as mips_topk; INVALID_ARG for a NULL or misaligned masks, nmasks < 1 or
 * mask_words < ceil(n/32); UNSUPPORTED for nmasks > MIPS_MAX_MASKS or b * nmasks >
 * MIPS_B_MAX.
 */
#define MIPS_MAX_MASKS 4
MIPS_API size_t mips_topk_masks_workspace_size(int32_t b, int64_t n, int32_t d, int32_t k,
                                               int32_t query_dtype, int32_t corpus_dtype,
                                               int32_t nmasks, int64_t candidates_per_list);
MIPS_API int mips_topk_masks(const void *queries, int32_t query_dtype, int32_t b, const void *corpus,
                             const float *row_scale, int32_t corpus_dtype, int64_t n, int32_t d,
                             const uint32_t *masks, int32_t nmasks, int64_t mask_words, int32_t k,
                             float *out_scores, int32_t *out_ids, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * mips_type_bitmap -- the exclusion bitmap of a search restricted to one item type: id i
 * is excluded when item_types[i] != target or exclude marks it (the per-type mask of
 * `RecsysTwoTowerModel.forward`, recsys_two_tower_model.py, one result set per target
 * type). Feed the result to mips_topk, or one row per type to mips_topk_masks; excluded
 * ids are never returned, so every id a type-restricted search returns has that type.
 *   item_types   device int32 [n]; n >= 1.
 *   exclude      device uint32 [ceil(n/32)] or NULL: ids excluded in any case.
 *   out_bitmap   device uint32 [ceil(n/32)]; bits of ids >= n are set. May alias exclude.
 * Errors: INVALID_ARG (NULL, n < 1, misaligned pointers), HIP (the launch failed).
 */
MIPS_API int mips_type_bitmap(const int32_t *item_types, int64_t n, int32_t target,
                              const uint32_t *exclude, uint32_t *out_bitmap, void *stream);

/*
 * mips_merge_topk -- merge of p sorted result lists per query into one top-k_out: the
 * fresh-shard pattern of "Two-Tower Retrieval at Industrial Scale" (engineeringmaxxing.com:
 * a small fresh index is searched beside the base index and the result lists are merged
 * by score), and the exchange step of a corpus split by rows across devices.
 *   in_scores    device float [p, b, k_in] (list-major): list l, query q, rank j.
 *   in_ids       device int32 [p, b, k_in]: ids local to list l's index; id < 0 is
 *                padding and is skipped (as mips_topk pads with (-INFINITY, -1)).
 *   offsets      host int64 [p], each in [0, 2^31): list l's ids are shifted by
 *                offsets[l]. Shifted ids must be distinct across lists (disjoint
 *                indexes) and below 2^31.
 *   p            1 .. 64 lists; b 1 .. MIPS_B_MAX queries; k_in >= 1; k_out 1 .. MIPS_K_MAX.
 *   out_scores   device float [b, k_out]; out_ids device int32 [b, k_out]: per query the
 *                k_out best real entries of all lists, score descending then id
 *                ascending, then (-INFINITY, -1). Exact for its inputs: when each list is
 *                its index's exact top-k_out, the result is the exact top-k_out of the
 *                union of the indexes.
 * Errors: INVALID_ARG (NULL, p/b/k out of range, an offset out of range, misaligned
 * pointers), UNSUPPORTED (k_out > MIPS_K_MAX or b > MIPS_B_MAX), HIP (the launch failed).
 */
MIPS_API int mips_merge_topk(const float *in_scores, const int32_t *in_ids, const int64_t *offsets,
                             int32_t p, int32_t b, int32_t k_in, int32_t k_out, float *out_scores,
                             int32_t *out_ids, void *stream);

/*
 * mips_merge_interests -- per user, the merge of its m interest vectors' result lists:
 * a user with several interest vectors matches an item by the best of them ("Two-Tower
 * Retrieval at Industrial Scale", engineeringmaxxing.com, section "Beyond Dot Products":
 * one search per interest vector, results merged by the maximum). An id returned for
 * several of the user's vectors keeps its highest score; the best k_out ids follow, score
 * descending then id ascending, then (-INFINITY, -1). When each list is its vector's exact
 * top-k_out (mips_topk over the b * m vectors), the result is the exact top-k_out by the
 * maximum over the user's vectors.
 *   in_scores    device float [b, m, k_in] (user-major: rows u*m .. u*m+m-1 of a mips_topk
 *                output); in_ids device int32 [b, m, k_in], id < 0 is padding.
 *   b 1 .. MIPS_B_MAX users, m >= 1 vectors per user, k_in >= 1 with m * k_in <= 2048,
 *   k_out 1 .. MIPS_K_MAX.
 *   out_scores   device float [b, k_out]; out_ids device int32 [b, k_out].
 * Errors: INVALID_ARG (NULL, b/m/k < 1, misaligned pointers), UNSUPPORTED (m * k_in > 2048,
 * k_out > MIPS_K_MAX or b > MIPS_B_MAX), HIP (the launch failed).
 */
MIPS_API int mips_merge_interests(const float *in_scores, const int32_t *in_ids, int32_t b, int32_t m,
                                  int32_t k_in, int32_t k_out, float *out_scores, int32_t *out_ids,
                                  void *stream);

/*
 * mips_set_timing_events -- profiling hook (host, per calling thread). When both are
 * non-NULL, later mips_topk calls on this thread launch the main score kernel so that its
 * dispatch records `before` (a hipEvent_t) at the kernel's start and `after` at its end,
 * on the call's stream (no packets of their own, so no gap between the call's kernels).
 * Pass NULL, NULL to stop. Returns MIPS_OK.
 */
MIPS_API int mips_set_timing_events(void *before, void *after);

/* Human-readable name of a status code (host, static storage). */
MIPS_API const char *mips_status_string(int status);

/* HIP error code of the last MIPS_ERR_HIP returned on this thread (host). */
MIPS_API int mips_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MIPS_H */
