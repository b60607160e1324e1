"""CPU oracle for exhaustive inner-product top-K (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package. It wraps `mips_oracle.c` (plain C, fp64, full sort) through ctypes and
shares no code with the HIP library.

Functions take and return numpy arrays:

* ``prepare(x, dtype)`` -- normalise raw fp32 rows in binary32 (the precision of the
  Model's float32 tensors) and pack them row-major, every code decided from that value
  (``"f32"`` -> float32, ``"bf16"`` -> uint16 codes, ``"fp8"`` -> uint8 E4M3 codes plus a
  float32 per-row power-of-two scale, ``"int8"`` -> int8 codes plus a float32 per-row
  scale max|y|/127).
* ``normalize(x)`` -- the fp64 normalised rows.
* ``topk(queries, q_dtype, corpus, c_dtype, k, row_scale=None, exclude=None)`` --
  fp64 scores [b, k] and int32 ids [b, k], sorted by score descending then id ascending.
* ``scores(...)`` -- exact scores of given (query, id) pairs.
* ``topk_int8(queries, q_dtype, corpus, k, row_scale, exclude=None)`` and
  ``scores_int8(...)`` -- the quantised scoring branch against an int8 index, step by step
  in binary32 (per-query int8 codes with scale max|u|/127, exact integer dot products,
  then the query scale, then the row scale).
* ``quantize(x, x_dtype, dtype)`` -- rows as given (no normalisation) quantised to
  ``"int8"`` (the per-query rule above) or ``"fp8"`` (E4M3 with a power-of-two scale).
* ``merge_topk(scores, ids, offsets, k)`` -- merge of per-index sorted result lists
  ([p, b, k_in]) into one top-k per query, ids shifted by each index's offset.
* ``maxsim_topk(queries [b, m, d], ...)`` -- top-k of users with m interest vectors each,
  an item scored by its best match over the user's vectors (``maxsim_topk_int8``: against
  an int8 index by the quantised branch).
* ``e4m3_value``, ``bf16_value``, ``bf16_from``, ``e4m3_from``, ``e4m3_row_scale``,
  ``i8_from``, ``i8_row_scale`` -- the scalar format helpers, exposed for the format pins.
"""
from __future__ import annotations

import concurrent.futures as _cf
import ctypes as C
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mips_oracle.c")
_LIB = os.path.join(_HERE, "libmips_oracle.so")

DTYPES = {"f32": 0, "bf16": 1, "fp8": 2, "int8": 3}
_CODE_TYPES = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "int8": np.int8}
_SCALED = ("fp8", "int8")
_STATUS = {0: "ok", 1: "bad argument", 2: "non-finite input", 3: "out of memory"}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C99, fp contraction off)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC",
                               "-shared", "-pthread", "-D_GNU_SOURCE", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = C.CDLL(_LIB)
        p = C.c_void_p
        i32, i64 = C.c_int32, C.c_int64
        L.oracle_bf16_value.argtypes = [C.c_uint16]
        L.oracle_bf16_value.restype = C.c_double
        L.oracle_e4m3_value.argtypes = [C.c_uint8]
        L.oracle_e4m3_value.restype = C.c_double
        L.oracle_bf16_from_f64.argtypes = [C.c_double]
        L.oracle_bf16_from_f64.restype = C.c_uint16
        L.oracle_e4m3_from_f64.argtypes = [C.c_double]
        L.oracle_e4m3_from_f64.restype = C.c_uint8
        L.oracle_e4m3_row_scale.argtypes = [C.c_double]
        L.oracle_e4m3_row_scale.restype = C.c_double
        L.oracle_i8_from_f64.argtypes = [C.c_double]
        L.oracle_i8_from_f64.restype = C.c_int8
        L.oracle_i8_row_scale.argtypes = [C.c_double]
        L.oracle_i8_row_scale.restype = C.c_double
        L.oracle_l2_normalize.argtypes = [p, i64, i32, p]
        L.oracle_prepare.argtypes = [p, i64, i32, i32, p, p]
        L.oracle_topk.argtypes = [i32, p, i32, i32, p, p, i64, i32, p, i32, p, p, i32]
        L.oracle_scores.argtypes = [i32, p, i32, i32, p, p, i64, i32, p, p, i64, p]
        L.oracle_merge_topk.argtypes = [p, p, p, i32, i32, i32, i32, p, p]
        L.oracle_quantize.argtypes = [i32, p, i64, i32, i32, p, p]
        L.oracle_topk_int8.argtypes = [i32, p, i32, p, p, i64, i32, p, i32, p, p, i32]
        L.oracle_scores_int8.argtypes = [i32, p, i32, p, p, i64, i32, p, p, i64, p]
        L.oracle_maxsim_topk_int8.argtypes = [i32, p, i32, i32, p, p, i64, i32, p, i32, p, p, i32]
        L.oracle_maxsim_topk.argtypes = [i32, p, i32, i32, i32, p, p, i64, i32, p, i32, p, p, i32]
        for f in (L.oracle_l2_normalize, L.oracle_prepare, L.oracle_topk, L.oracle_scores,
                  L.oracle_merge_topk, L.oracle_maxsim_topk, L.oracle_quantize,
                  L.oracle_topk_int8, L.oracle_scores_int8, L.oracle_maxsim_topk_int8):
            f.restype = C.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: {_STATUS.get(rc, rc)}")


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


# ----------------------------------------------------------------- scalars
def bf16_value(code: int) -> float:
    return lib().oracle_bf16_value(int(code))


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def bf16_from(v: float) -> int:
    return int(lib().oracle_bf16_from_f64(float(v)))


def e4m3_from(v: float) -> int:
    return int(lib().oracle_e4m3_from_f64(float(v)))


def e4m3_row_scale(amax: float) -> float:
    return lib().oracle_e4m3_row_scale(float(amax))


def i8_from(v: float) -> int:
    return int(lib().oracle_i8_from_f64(float(v)))


def i8_row_scale(amax: float) -> float:
    return lib().oracle_i8_row_scale(float(amax))


def decode(codes: np.ndarray, dtype: str, row_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 values of stored operands (rows scaled for fp8 and int8)."""
    if dtype == "f32":
        return np.asarray(codes, np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(codes, np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    if dtype == "int8":
        v = np.asarray(codes, np.int8).astype(np.float64)
    else:
        table = np.array([e4m3_value(c) for c in range(256)], np.float64)
        v = table[np.asarray(codes, np.uint8)]
    if row_scale is not None:
        v = v * np.asarray(row_scale, np.float64)[:, None]
    return v


# ----------------------------------------------------------------- arrays
def normalize(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    rows, d = x.shape
    y = np.empty((rows, d), np.float64)
    _check(lib().oracle_l2_normalize(_ptr(x), rows, d, _ptr(y)), "normalize")
    return y


def prepare(x: np.ndarray, dtype: str) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    x = np.ascontiguousarray(x, np.float32)
    rows, d = x.shape
    out = np.empty((rows, d), _CODE_TYPES[dtype])
    scale = np.empty(rows, np.float32) if dtype in _SCALED else None
    _check(lib().oracle_prepare(_ptr(x), rows, d, DTYPES[dtype], _ptr(out), _ptr(scale)),
           "prepare")
    return out, scale


def prepare_chunks(chunks, n: int, d: int, dtype: str, threads: Optional[int] = None
                   ) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """prepare() of a corpus given as (row0, raw rows) chunks, in parallel threads."""
    codes = np.empty((n, d), _CODE_TYPES[dtype])
    scale = np.empty(n, np.float32) if dtype in _SCALED else None

    def work(item):
        r0, blk = item
        c, s = prepare(blk, dtype)
        codes[r0:r0 + blk.shape[0]] = c
        if scale is not None:
            scale[r0:r0 + blk.shape[0]] = s

    nt = threads or min(16, default_threads())
    with _cf.ThreadPoolExecutor(nt) as ex:
        pending = []
        for it in chunks:
            pending.append(ex.submit(work, it))
            if len(pending) >= nt:          # bound the raw chunks held in memory
                pending.pop(0).result()
        for f in pending:
            f.result()
    return codes, scale


def topk(queries: np.ndarray, q_dtype: str, corpus: np.ndarray, c_dtype: str, k: int,
         row_scale: Optional[np.ndarray] = None, exclude: Optional[np.ndarray] = None,
         threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    queries = np.ascontiguousarray(queries)
    corpus = np.ascontiguousarray(corpus)
    b, d = queries.shape
    n = corpus.shape[0]
    assert corpus.shape[1] == d
    if row_scale is not None:
        row_scale = np.ascontiguousarray(row_scale, np.float32)
    if exclude is not None:
        exclude = np.ascontiguousarray(exclude, np.uint32)
        assert exclude.size >= (n + 31) // 32
    out_s = np.empty((b, k), np.float64)
    out_i = np.empty((b, k), np.int32)
    _check(lib().oracle_topk(DTYPES[q_dtype], _ptr(queries), b, DTYPES[c_dtype], _ptr(corpus),
                             _ptr(row_scale), n, d, _ptr(exclude), k, _ptr(out_s), _ptr(out_i),
                             threads or default_threads()), "topk")
    return out_s, out_i


def scores(queries: np.ndarray, q_dtype: str, corpus: np.ndarray, c_dtype: str,
           qidx: np.ndarray, ids: np.ndarray, row_scale: Optional[np.ndarray] = None
           ) -> np.ndarray:
    queries = np.ascontiguousarray(queries)
    corpus = np.ascontiguousarray(corpus)
    b, d = queries.shape
    n = corpus.shape[0]
    qidx = np.ascontiguousarray(qidx, np.int32).ravel()
    ids = np.ascontiguousarray(ids, np.int32).ravel()
    if row_scale is not None:
        row_scale = np.ascontiguousarray(row_scale, np.float32)
    out = np.empty(qidx.size, np.float64)
    _check(lib().oracle_scores(DTYPES[q_dtype], _ptr(queries), b, DTYPES[c_dtype], _ptr(corpus),
                               _ptr(row_scale), n, d, _ptr(qidx), _ptr(ids), qidx.size,
                               _ptr(out)), "scores")
    return out


def quantize(x: np.ndarray, x_dtype: str, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """Rows as given ([rows, d] f32 values, or bf16 codes with x_dtype "bf16") quantised
    without normalisation: (codes [rows, d], scale float32 [rows])."""
    x = np.ascontiguousarray(x)
    rows, d = x.shape
    codes = np.empty((rows, d), _CODE_TYPES[dtype])
    scale = np.empty(rows, np.float32)
    _check(lib().oracle_quantize(DTYPES[x_dtype], _ptr(x), rows, d, DTYPES[dtype], _ptr(codes),
                                 _ptr(scale)), "quantize")
    return codes, scale


def topk_int8(queries: np.ndarray, q_dtype: str, corpus: np.ndarray, k: int,
              row_scale: np.ndarray, exclude: Optional[np.ndarray] = None,
              threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k against an int8 index by the quantised scoring branch: binary32 scores [b, k]
    (as float64, exactly) and int32 ids [b, k], score descending then id ascending."""
    queries = np.ascontiguousarray(queries)
    corpus = np.ascontiguousarray(corpus, np.int8)
    b, d = queries.shape
    n = corpus.shape[0]
    assert corpus.shape[1] == d
    row_scale = np.ascontiguousarray(row_scale, np.float32)
    if exclude is not None:
        exclude = np.ascontiguousarray(exclude, np.uint32)
        assert exclude.size >= (n + 31) // 32
    out_s = np.empty((b, k), np.float64)
    out_i = np.empty((b, k), np.int32)
    _check(lib().oracle_topk_int8(DTYPES[q_dtype], _ptr(queries), b, _ptr(corpus),
                                  _ptr(row_scale), n, d, _ptr(exclude), k, _ptr(out_s),
                                  _ptr(out_i), threads or default_threads()), "topk_int8")
    return out_s, out_i


def scores_int8(queries: np.ndarray, q_dtype: str, corpus: np.ndarray, row_scale: np.ndarray,
                qidx: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Quantised-branch binary32 scores (as float64) of given (query, id) pairs."""
    queries = np.ascontiguousarray(queries)
    corpus = np.ascontiguousarray(corpus, np.int8)
    b, d = queries.shape
    n = corpus.shape[0]
    qidx = np.ascontiguousarray(qidx, np.int32).ravel()
    ids = np.ascontiguousarray(ids, np.int32).ravel()
    row_scale = np.ascontiguousarray(row_scale, np.float32)
    out = np.empty(qidx.size, np.float64)
    _check(lib().oracle_scores_int8(DTYPES[q_dtype], _ptr(queries), b, _ptr(corpus),
                                    _ptr(row_scale), n, d, _ptr(qidx), _ptr(ids), qidx.size,
                                    _ptr(out)), "scores_int8")
    return out


def merge_topk(scores: np.ndarray, ids: np.ndarray, offsets, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """scores float32 / ids int32 [p, b, k_in]; offsets int64 [p]."""
    scores = np.ascontiguousarray(scores, np.float32)
    ids = np.ascontiguousarray(ids, np.int32)
    p, b, k_in = scores.shape
    offsets = np.ascontiguousarray(offsets, np.int64)
    assert offsets.size == p and ids.shape == scores.shape
    out_s = np.empty((b, k), np.float32)
    out_i = np.empty((b, k), np.int32)
    _check(lib().oracle_merge_topk(_ptr(scores), _ptr(ids), _ptr(offsets), p, b, k_in, k,
                                   _ptr(out_s), _ptr(out_i)), "merge_topk")
    return out_s, out_i


def maxsim_topk(queries: np.ndarray, q_dtype: str, corpus: np.ndarray, c_dtype: str, k: int,
                row_scale: Optional[np.ndarray] = None, exclude: Optional[np.ndarray] = None,
                threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """queries [b, m, d]: fp64 max-over-vectors scores [b, k] and ids [b, k]."""
    queries = np.ascontiguousarray(queries)
    corpus = np.ascontiguousarray(corpus)
    b, m, d = queries.shape
    n = corpus.shape[0]
    if row_scale is not None:
        row_scale = np.ascontiguousarray(row_scale, np.float32)
    if exclude is not None:
        exclude = np.ascontiguousarray(exclude, np.uint32)
    out_s = np.empty((b, k), np.float64)
    out_i = np.empty((b, k), np.int32)
    _check(lib().oracle_maxsim_topk(DTYPES[q_dtype], _ptr(queries), b, m, DTYPES[c_dtype],
                                    _ptr(corpus), _ptr(row_scale), n, d, _ptr(exclude), k,
                                    _ptr(out_s), _ptr(out_i), threads or default_threads()),
           "maxsim_topk")
    return out_s, out_i


def maxsim_topk_int8(queries: np.ndarray, q_dtype: str, corpus: np.ndarray, k: int,
                     row_scale: np.ndarray, exclude: Optional[np.ndarray] = None,
                     threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """maxsim_topk against an int8 index, each vector scored by the quantised branch."""
    queries = np.ascontiguousarray(queries)
    corpus = np.ascontiguousarray(corpus, np.int8)
    b, m, d = queries.shape
    n = corpus.shape[0]
    row_scale = np.ascontiguousarray(row_scale, np.float32)
    if exclude is not None:
        exclude = np.ascontiguousarray(exclude, np.uint32)
    out_s = np.empty((b, k), np.float64)
    out_i = np.empty((b, k), np.int32)
    _check(lib().oracle_maxsim_topk_int8(DTYPES[q_dtype], _ptr(queries), b, m, _ptr(corpus),
                                         _ptr(row_scale), n, d, _ptr(exclude), k, _ptr(out_s),
                                         _ptr(out_i), threads or default_threads()),
           "maxsim_topk_int8")
    return out_s, out_i
