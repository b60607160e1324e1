"""Test helpers: the top-K acceptance rule, the packed-layout decoder and input builders.

The layout decoder follows the byte-layout formula written in include/mips.h; it is test
code and does not import anything from the library.
"""
from __future__ import annotations

import os
from typing import Optional

import numpy as np

import oracle

# int8 is checked against the oracle's quantised branch instead (check_int8): identical
# results on identical codes, else one code step per row. The entry below is the bound of
# the quantised score against the exact score of the unquantised query, max|q| ||c||_1 / 254
# <= sqrt(D) / 254 (0.063 at D = 256), used where a test compares with exact scores.
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "int8": 6e-2}
# Expected error floors: fp32 accumulation of the same stored operands (f32, bf16) and
# E4M3 quantisation of the queries (fp8). Far above these means a bug even inside TOL.
# A bf16 index also gets one code step per returned row (check_topk): the GPU and the
# oracle both normalise rows in binary32 but sum the squares in different orders, so about
# one stored element in 10^5 rounds to the neighbouring bf16 code; one step of element d
# moves a score by |q_d| ulp(c_d), at most 2^-7 |q_d c_d| (8 significant bits).
FLOOR = {"f32": 2e-6, "bf16": 5e-4, "fp8": 3e-2, "int8": 1e-2}


def floor_for(c_dtype: str, q_dtype: str) -> float:
    """f32 queries against a bf16 corpus are rounded to bf16 on the GPU (the oracle keeps
    them): each term moves by at most 2^-9 of |q_d c_d|, so the score by at most ~2^-9."""
    if c_dtype == "bf16" and q_dtype == "f32":
        return 2.0 ** -9 + FLOOR["bf16"]
    return FLOOR[c_dtype]


def threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


# ------------------------------------------------------------------- layout
def untile(packed: np.ndarray, n: int, d: int, dtype: str) -> np.ndarray:
    """Logical row-major [n, d] element codes of a fragment-tiled buffer (include/mips.h)."""
    E = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1}[dtype]
    per = 16 // E
    nblk = (n + 31) // 32
    buf = np.asarray(packed, np.uint8)[: nblk * 32 * d * E]
    elem = buf.view({"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8, "int8": np.int8}[dtype])
    nch = 32 * d * E // 1024
    elem = elem.reshape(nblk, nch, 64, per)
    c = np.arange(nch)[:, None, None]
    s = np.arange(64)[None, :, None]
    t = np.arange(per)[None, None, :]
    h = s >> 5
    if dtype == "f32":
        dim = 8 * c + 2 * t + h
    elif dtype == "bf16":
        dim = 16 * c + 8 * h + t
    elif dtype == "int8":
        dim = 32 * c + 16 * h + t
    else:
        dim = 64 * (c >> 1) + 32 * h + 16 * (c & 1) + t
    row = np.broadcast_to(s & 31, dim.shape)
    out = np.empty((nblk, 32, d), elem.dtype)
    out[:, row.ravel(), dim.ravel()] = elem.reshape(nblk, -1)
    out = out.reshape(nblk * 32, d)[:n]
    return out.view(np.float32) if dtype == "f32" else out


def tile(codes: np.ndarray, dtype: str) -> np.ndarray:
    """Fragment-tiled bytes (include/mips.h) of row-major [n, d] codes, the inverse of
    untile; rows past n up to the block size are zero."""
    n, d = codes.shape
    E = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1}[dtype]
    per = 16 // E
    nblk = (n + 31) // 32
    et = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8, "int8": np.uint8}[dtype]
    src = np.zeros((nblk * 32, d), et)
    src[:n] = np.ascontiguousarray(codes).view(et)
    src = src.reshape(nblk, 32, d)
    nch = 32 * d * E // 1024
    c = np.arange(nch)[:, None, None]
    s = np.arange(64)[None, :, None]
    t = np.arange(per)[None, None, :]
    h = s >> 5
    if dtype == "f32":
        dim = 8 * c + 2 * t + h
    elif dtype == "bf16":
        dim = 16 * c + 8 * h + t
    elif dtype == "int8":
        dim = 32 * c + 16 * h + t
    else:
        dim = 64 * (c >> 1) + 32 * h + 16 * (c & 1) + t
    row = np.broadcast_to(s & 31, dim.shape)
    out = src[:, row.ravel(), dim.ravel()].reshape(nblk, nch, 64, per)
    return np.ascontiguousarray(out).view(np.uint8).ravel()


def upload_corpus(codes: np.ndarray, scale: Optional[np.ndarray], dtype: str, dev):
    """A library corpus holding exactly the given row-major codes (and row scales), packed
    on the host: the GPU then searches the very operands the oracle scores."""
    import torch

    import exact_inner_product_amd as mips
    n, d = codes.shape
    packed = torch.from_numpy(tile(codes, dtype)).to(dev)
    assert packed.numel() == mips.corpus_bytes(n, d, dtype)
    rs = None
    if dtype in ("fp8", "int8"):
        full = np.full((n + 31) // 32 * 32, 1.0 if dtype == "fp8" else np.float32(1e-12), np.float32)
        full[:n] = scale
        rs = torch.from_numpy(full).to(dev)
    return mips.Corpus(packed, rs, n, d, dtype)


def query_tensor(codes: np.ndarray, dtype: str, dev):
    """Query codes from the oracle side as the device tensor the library takes."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(codes).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(codes, np.float32)).to(dev)


# ------------------------------------------------------------------ references
def ref_topk(q_codes, q_dtype, c_codes, c_dtype, k, row_scale=None, exclude=None, threads=None):
    """The oracle's top-k for this dtype: the quantised scoring branch for an int8 index,
    the exact fp64 scores otherwise."""
    if c_dtype == "int8":
        return oracle.topk_int8(q_codes, q_dtype, c_codes, k, row_scale, exclude=exclude,
                                threads=threads)
    return oracle.topk(q_codes, q_dtype, c_codes, c_dtype, k, row_scale=row_scale,
                       exclude=exclude, threads=threads)


def ref_scores(q_codes, q_dtype, c_codes, c_dtype, qidx, ids, row_scale=None):
    if c_dtype == "int8":
        return oracle.scores_int8(q_codes, q_dtype, c_codes, row_scale, qidx, ids)
    return oracle.scores(q_codes, q_dtype, c_codes, c_dtype, qidx, ids, row_scale=row_scale)


# ---------------------------------------------------------------- acceptance
def check_topk(g_scores: np.ndarray, g_ids: np.ndarray, o_scores: np.ndarray, o_ids: np.ndarray,
               q_codes: np.ndarray, q_dtype: str, c_codes: np.ndarray, c_dtype: str,
               row_scale: Optional[np.ndarray], excluded: Optional[set], n: int, tau: float,
               floor: Optional[float] = None) -> dict:
    """Acceptance rule for each query row: well-formed output, score errors and the score
    profile within tau, id sets equal except swaps within tau of the K-th score.

    o_scores/o_ids: the oracle's exact top-K of the same queries (q_codes). Returns stats.
    """
    if c_dtype == "int8":
        return check_int8(g_scores, g_ids, o_scores, o_ids, q_codes, q_dtype, c_codes,
                          row_scale, excluded, n)
    b, k = g_ids.shape
    excluded = excluded or set()
    eligible = n - len(excluded)
    kk = min(k, eligible)
    stats = {"max_err": 0.0, "max_profile": 0.0, "swaps": 0}
    for qi in range(b):
        gi, gs = g_ids[qi], g_scores[qi]
        # 1. well-formed
        ids, sc = _well_formed(qi, gi, gs, kk, n, excluded)
        if kk == 0:
            continue
        # 2. score error against the exact score of the returned id
        e = oracle.scores(q_codes, q_dtype, c_codes, c_dtype, np.full(kk, qi), ids,
                          row_scale=row_scale)
        err = np.abs(sc - e).max()
        stats["max_err"] = max(stats["max_err"], float(err))
        assert err <= tau, f"query {qi}: score error {err} > {tau}"
        if floor is not None:
            allow = np.full(kk, floor)
            if c_dtype == "bf16":
                qv = oracle.decode(q_codes[qi], q_dtype)
                cv = oracle.decode(c_codes[ids], c_dtype)
                allow += 2.0 ** -7 * np.abs(cv * qv).max(axis=1)
            over = np.abs(sc - e) - allow
            stats["max_over_floor"] = max(stats.get("max_over_floor", -np.inf), float(over.max()))
        # 3. profile
        prof = np.abs(sc - o_scores[qi, :kk]).max()
        stats["max_profile"] = max(stats["max_profile"], float(prof))
        assert prof <= tau, f"query {qi}: profile error {prof} > {tau}"
        # 4. id sets
        diff = set(ids.tolist()) ^ set(o_ids[qi, :kk].tolist())
        if diff:
            dl = np.array(sorted(diff), np.int32)
            ed = oracle.scores(q_codes, q_dtype, c_codes, c_dtype, np.full(dl.size, qi), dl,
                               row_scale=row_scale)
            assert np.all(np.abs(ed - o_scores[qi, kk - 1]) <= tau), \
                f"query {qi}: id swap beyond tolerance"
            stats["swaps"] += len(diff) // 2
    if floor is not None:
        assert stats.get("max_over_floor", -np.inf) <= 0.0, \
            f"error {stats['max_err']} far above the expected floor {floor} (+ one bf16 step)"
    return stats


def _well_formed(qi, gi, gs, kk, n, excluded):
    """K' distinct ids in [0, n), none excluded, sorted by (score desc, id asc), then
    exactly (-inf, -1) padding. Returns the K' ids and scores."""
    assert np.all(gi[kk:] == -1) and np.all(np.isneginf(gs[kk:])), (qi, gi[kk:], gs[kk:])
    ids = gi[:kk]
    assert np.all((ids >= 0) & (ids < n)), qi
    assert len(set(ids.tolist())) == kk, "duplicate ids"
    assert not (set(ids.tolist()) & excluded), "excluded id returned"
    sc = gs[:kk]
    assert np.all(np.isfinite(sc))
    order_ok = (sc[:-1] > sc[1:]) | ((sc[:-1] == sc[1:]) & (ids[:-1] < ids[1:]))
    assert np.all(order_ok), "GPU list not sorted by (score desc, id asc)"
    return ids, sc


def int8_step(q_codes: np.ndarray, q_dtype: str, row_scale: np.ndarray, qi: int, ids) -> np.ndarray:
    """Largest move of a returned row's quantised score when one element of the row's int8
    codes sits one step away (the GPU and the oracle build the index in binary32 but sum
    the squares in different orders): us * 127 * s_id, i.e. max|u| s_id, plus rounding."""
    u = oracle.decode(q_codes[qi:qi + 1], q_dtype)[0].astype(np.float32)
    us = max(float(np.float32(np.abs(u).max()) / np.float32(127.0)), float(np.float32(1e-12)))
    return us * 127.0 * np.asarray(row_scale, np.float64)[ids] * (1 + 2.0 ** -20)


def check_int8(g_scores, g_ids, o_scores, o_ids, q_codes, q_dtype, c_codes, row_scale,
               excluded, n, exact: bool = False) -> dict:
    """Acceptance rule of an int8 index against the oracle's quantised scoring branch
    (oracle.topk_int8 / scores_int8: per-query int8 codes, exact integer dot products, then
    the query scale and the row scale in binary32).

    exact=True (the GPU searched the oracle's own codes): ids and binary32 scores must be
    identical. Otherwise (each side built its own index): every returned score is within one
    code step of its row's oracle score (int8_step), the score profile likewise, and the id
    sets agree except swaps within two steps of the oracle's K-th score."""
    b, k = g_ids.shape
    excluded = excluded or set()
    kk = min(k, n - len(excluded))
    stats = {"max_err": 0.0, "max_profile": 0.0, "swaps": 0, "exact_rows": 0}
    for qi in range(b):
        ids, sc = _well_formed(qi, g_ids[qi], g_scores[qi], kk, n, excluded)
        if kk == 0:
            continue
        if exact:
            assert np.array_equal(ids, o_ids[qi, :kk]), f"query {qi}: ids differ from the oracle"
            assert np.array_equal(sc.astype(np.float32).view(np.uint32),
                                  o_scores[qi, :kk].astype(np.float32).view(np.uint32)), \
                f"query {qi}: scores differ from the oracle"
            stats["exact_rows"] += 1
            continue
        e = oracle.scores_int8(q_codes, q_dtype, c_codes, row_scale, np.full(kk, qi), ids)
        err = np.abs(sc - e)
        allow = int8_step(q_codes, q_dtype, row_scale, qi, ids)
        stats["max_err"] = max(stats["max_err"], float(err.max()))
        assert np.all(err <= allow), f"query {qi}: score beyond one code step of the oracle's"
        stats["exact_rows"] += int(np.all(err == 0))
        prof = np.abs(sc - o_scores[qi, :kk]).max()
        stats["max_profile"] = max(stats["max_profile"], float(prof))
        assert prof <= allow.max() * 2, f"query {qi}: profile error {prof}"
        diff = set(ids.tolist()) ^ set(o_ids[qi, :kk].tolist())
        if diff:
            dl = np.array(sorted(diff), np.int32)
            ed = oracle.scores_int8(q_codes, q_dtype, c_codes, row_scale, np.full(dl.size, qi), dl)
            lim = 2 * int8_step(q_codes, q_dtype, row_scale, qi, dl)
            assert np.all(np.abs(ed - o_scores[qi, kk - 1]) <= lim), \
                f"query {qi}: id swap beyond two code steps"
            stats["swaps"] += len(diff) // 2
    return stats


def operand_queries(q_codes: np.ndarray, q_dtype: str, c_dtype: str):
    """The query operand the GPU multiplies, as oracle-side codes: bf16 for a bf16 index
    (f32 queries are rounded to nearest even), E4M3 times the query's power-of-two scale
    for an fp8 index (exactly an f32 value), the queries themselves for an f32 index.
    Returns (codes, dtype) for oracle.topk / oracle.scores."""
    if c_dtype == "bf16" and q_dtype == "f32":
        v = np.asarray(q_codes, np.float32)
        return np.vectorize(oracle.bf16_from, otypes=[np.uint16])(v.astype(np.float64)), "bf16"
    if c_dtype == "fp8":
        q8, s8 = oracle.quantize(q_codes, q_dtype, "fp8")
        return (oracle.decode(q8, "fp8") * s8[:, None].astype(np.float64)).astype(np.float32), "f32"
    return q_codes, q_dtype


def operand_reference(q_codes, q_dtype, c_codes, c_dtype, k, row_scale=None, exclude=None,
                      threads_=None):
    """The oracle's top-k of the operands the GPU multiplies (int8: the quantised branch)."""
    if c_dtype == "int8":
        return oracle.topk_int8(q_codes, q_dtype, c_codes, k, row_scale, exclude=exclude,
                                threads=threads_)
    q_op, q_op_dt = operand_queries(q_codes, q_dtype, c_dtype)
    return oracle.topk(q_op, q_op_dt, c_codes, c_dtype, k, row_scale=row_scale, exclude=exclude,
                       threads=threads_)


def operands_are_inputs(q_dtype: str, c_dtype: str) -> bool:
    """True when the GPU multiplies the queries as given (its operand reference is then
    also the end-to-end reference)."""
    return c_dtype == "int8" or q_dtype == c_dtype or (c_dtype == "bf16" and q_dtype == "bf16")


# The E4M3 MFMA with block scales (v_mfma_scale_f32_32x32x64_f8f6f4) sums its products with
# less than binary32 precision: the OCP microscaling format leaves the internal precision of
# a scaled dot product to the implementation. Measured on gfx950 against the exact score of
# its operands (D = 64..256, 60K rows x 64 queries x 1024 results each): at most
# 803 * 2^-24 sum_d |q_d c_d|, about 2^-14.3. The fp8 check allows 2^-11 sum_d |q_d c_d|.
FP8_MFMA_REL = 2.0 ** -11


def accumulation_bound(q_op, q_op_dtype, c_codes, c_dtype, row_scale, qi, ids) -> np.ndarray:
    """Bound on the GPU's accumulation of D products of stored operands: for binary32, in any
    order and with each product rounded at most once, (D + 2) 2^-24 sum_d |q_d c_d|; for the
    scaled fp8 MFMA, FP8_MFMA_REL sum_d |q_d c_d|."""
    qv = oracle.decode(q_op[qi:qi + 1], q_op_dtype)[0]
    cv = oracle.decode(c_codes[ids], c_dtype,
                       None if row_scale is None else np.asarray(row_scale)[ids])
    d = qv.size
    rel = FP8_MFMA_REL if c_dtype == "fp8" else (d + 2) * 2.0 ** -24
    return rel * np.abs(cv * qv).sum(axis=1) + 1e-30


def check_operands(g_scores, g_ids, q_codes, q_dtype, c_codes, c_dtype, row_scale, excluded,
                   n, exclude_bitmap=None, threads_=None, ref=None) -> dict:
    """Parity of a search of the oracle's own codes (corpus and queries) against the exact
    scores of the operands the GPU multiplies (operand_queries): every returned score within
    the binary32 accumulation bound of its row's exact score, ids identical to the oracle's
    exact top-k except swaps within twice that bound of the K-th score. int8 goes to
    check_int8 with exact=True (identical codes give identical binary32 scores). ref: the
    oracle's top-k of the operands (operand_reference), if already computed."""
    b, k = g_ids.shape
    excluded = excluded or set()
    kk = min(k, n - len(excluded))
    if c_dtype == "int8":
        o_s, o_i = ref if ref is not None else oracle.topk_int8(
            q_codes, q_dtype, c_codes, k, row_scale, exclude=exclude_bitmap, threads=threads_)
        return check_int8(g_scores, g_ids, o_s, o_i, q_codes, q_dtype, c_codes, row_scale,
                          excluded, n, exact=True)
    q_op, q_op_dt = operand_queries(q_codes, q_dtype, c_dtype)
    if ref is None:
        ref = oracle.topk(q_op, q_op_dt, c_codes, c_dtype, k, row_scale=row_scale,
                          exclude=exclude_bitmap, threads=threads_)
    o_s, o_i = ref
    stats = {"max_err": 0.0, "max_rel_to_bound": 0.0, "swaps": 0}
    for qi in range(b):
        ids, sc = _well_formed(qi, g_ids[qi], g_scores[qi], kk, n, excluded)
        if kk == 0:
            continue
        e = oracle.scores(q_op, q_op_dt, c_codes, c_dtype, np.full(kk, qi), ids,
                          row_scale=row_scale)
        bound = accumulation_bound(q_op, q_op_dt, c_codes, c_dtype, row_scale, qi, ids)
        err = np.abs(sc - e)
        stats["max_err"] = max(stats["max_err"], float(err.max()))
        stats["max_rel_to_bound"] = max(stats["max_rel_to_bound"], float((err / bound).max()))
        assert np.all(err <= bound), f"query {qi}: error {err.max()} beyond the accumulation bound"
        diff = set(ids.tolist()) ^ set(o_i[qi, :kk].tolist())
        if diff:
            dl = np.array(sorted(diff), np.int32)
            ed = oracle.scores(q_op, q_op_dt, c_codes, c_dtype, np.full(dl.size, qi), dl,
                               row_scale=row_scale)
            # a swapped pair (g returned, o not) has e(o) - bound(o) <= s(o) <= s(g) <=
            # e(g) + bound(g), and e(g) <= e_K <= e(o)
            lim = 2 * max(bound.max(), accumulation_bound(q_op, q_op_dt, c_codes, c_dtype,
                                                          row_scale, qi, dl).max())
            assert np.all(np.abs(ed - o_s[qi, kk - 1]) <= lim), \
                f"query {qi}: id swap beyond the accumulation bound"
            stats["swaps"] += len(diff) // 2
    return stats


# ------------------------------------------------------------------- inputs
def oracle_corpus(w, chunk=1 << 20):
    """Oracle-side packed corpus (row-major codes) of workload w, prepared in parallel."""
    return oracle.prepare_chunks(w.corpus_chunks(chunk), w.n, w.d, w.corpus_dtype, threads())
