"""Test helpers: the top-K acceptance rule, the packed-layout decoder and input builders.

The layout decoder follows the byte-layout formula written in include/mips.h; it is test
code and does not import anything from the library.
"""
from __future__ import annotations

import os
from typing import Optional

import numpy as np

import oracle

# int8: the GPU quantises each query to int8 (scale max|q|/127); a term moves by at most
# half a step, so a score by at most max|q| * ||c||_1 / 254 <= sqrt(D) / 254 (0.063 at
# D = 256), the fp8 budget.
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


# ---------------------------------------------------------------- acceptance
def check_topk(g_scores: np.ndarray, g_ids: np.ndarray, o_scores: np.ndarray, o_ids: np.ndarray,
               q_codes: np.ndarray, q_dtype: str, c_codes: np.ndarray, c_dtype: str,
               row_scale: Optional[np.ndarray], excluded: Optional[set], n: int, tau: float,
               floor: Optional[float] = None) -> dict:
    """Acceptance rule for each query row: well-formed output, score errors and the score
    profile within tau, id sets equal except swaps within tau of the K-th score.

    o_scores/o_ids: the oracle's exact top-K of the same queries (q_codes). Returns stats.
    """
    b, k = g_ids.shape
    excluded = excluded or set()
    eligible = n - len(excluded)
    kk = min(k, eligible)
    stats = {"max_err": 0.0, "max_profile": 0.0, "swaps": 0}
    for qi in range(b):
        gi, gs = g_ids[qi], g_scores[qi]
        # 1. well-formed
        assert np.all(gi[kk:] == -1) and np.all(np.isneginf(gs[kk:])), (qi, gi[kk:], gs[kk:])
        ids = gi[:kk]
        assert np.all((ids >= 0) & (ids < n)), qi
        assert len(set(ids.tolist())) == kk, "duplicate ids"
        assert not (set(ids.tolist()) & excluded), "excluded id returned"
        sc = gs[:kk]
        assert np.all(np.isfinite(sc))
        order_ok = (sc[:-1] > sc[1:]) | ((sc[:-1] == sc[1:]) & (ids[:-1] < ids[1:]))
        assert np.all(order_ok), "GPU list not sorted by (score desc, id asc)"
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


# ------------------------------------------------------------------- inputs
def oracle_corpus(w, chunk=1 << 20):
    """Oracle-side packed corpus (row-major codes) of workload w, prepared in parallel."""
    return oracle.prepare_chunks(w.corpus_chunks(chunk), w.n, w.d, w.corpus_dtype, threads())
