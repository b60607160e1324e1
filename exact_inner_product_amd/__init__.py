"""Python binding of libmips, the gfx950 exhaustive inner-product top-K library.

Argument marshalling only: every step of the path runs in the HIP kernels behind the C ABI
declared in include/mips.h. PyTorch provides device memory and the current stream.
Importing works without a GPU; calling needs the built library (``python -m
exact_inner_product_amd.build``) and raises if it is missing.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmips.so")

F32, BF16, FP8_E4M3, INT8 = 0, 1, 2, 3
DTYPE_CODES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "int8": INT8}
SCALED = ("fp8", "int8")  # packed with one float scale per row
K_MAX = 1024
B_MAX = 1 << 23  # result lists per call (queries, or queries x masks)

EXPORTS = (
    "mips_corpus_bytes", "mips_scale_count", "mips_l2_normalize", "mips_prepare_corpus",
    "mips_topk_workspace_size", "mips_topk_workspace_size_for", "mips_topk", "mips_topk_noalloc",
    "mips_topk_ranges",
    "mips_topk_masks_workspace_size", "mips_topk_masks",
    "mips_merge_topk", "mips_merge_interests", "mips_type_bitmap", "mips_set_timing_events", "mips_status_string", "mips_last_hip_error",
)
MERGE_MAX_LISTS = 64
MAX_MASKS = 4  # result sets of one mips_topk_masks pass


class MipsError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib().mips_status_string(status).decode()
        if status == 4:
            msg += f" (hip error {lib().mips_last_hip_error()})"
        super().__init__(f"{what}: {msg}")


class VersionSkew(RuntimeError):
    """Queries from one model version against an index built by another: the scores would
    be noise, so the call is refused before any work is enqueued."""


_lib = None


def lib() -> C.CDLL:
    """The loaded libmips.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmips.so is not built ({LIB_PATH}); run "
                               "`python -m exact_inner_product_amd.build`")
        L = C.CDLL(LIB_PATH)
        p, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.mips_corpus_bytes.argtypes = [i64, i32, i32]
        L.mips_corpus_bytes.restype = i64
        L.mips_scale_count.argtypes = [i64]
        L.mips_scale_count.restype = i64
        L.mips_l2_normalize.argtypes = [p, i64, i32, i32, p, p]
        L.mips_prepare_corpus.argtypes = [p, i64, i64, i32, i32, p, p, p]
        L.mips_topk_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32]
        L.mips_topk_workspace_size.restype = sz
        L.mips_topk_workspace_size_for.argtypes = [i32, i64, i32, i32, i32, i32, i64]
        L.mips_topk_workspace_size_for.restype = sz
        L.mips_topk.argtypes = [p, i32, i32, p, p, i32, i64, i32, p, i64, i32, p, p, p, sz, p]
        L.mips_topk_noalloc.argtypes = [p, i32, i32, p, p, i32, i64, i32, p, i64, i32, p, p, p]
        L.mips_topk_ranges.argtypes = [p, i32, i32, p, p, i32, i64, i32, p, i64, p, i32, i32, p, p, p,
                                       sz, p]
        L.mips_topk_masks_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32, i64]
        L.mips_topk_masks_workspace_size.restype = sz
        L.mips_topk_masks.argtypes = [p, i32, i32, p, p, i32, i64, i32, p, i32, i64, i32, p, p, p,
                                      sz, p]
        L.mips_merge_topk.argtypes = [p, p, p, i32, i32, i32, i32, p, p, p]
        L.mips_merge_interests.argtypes = [p, p, i32, i32, i32, i32, p, p, p]
        L.mips_type_bitmap.argtypes = [p, i64, i32, p, p, p]
        L.mips_set_timing_events.argtypes = [p, p]
        L.mips_status_string.argtypes = [C.c_int]
        L.mips_status_string.restype = C.c_char_p
        L.mips_last_hip_error.argtypes = []
        for f in (L.mips_l2_normalize, L.mips_prepare_corpus, L.mips_topk, L.mips_topk_noalloc,
                  L.mips_topk_ranges,
                  L.mips_topk_masks,
                  L.mips_merge_topk, L.mips_merge_interests, L.mips_type_bitmap,
                  L.mips_set_timing_events, L.mips_last_hip_error):
            f.restype = C.c_int
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise MipsError(status, what)


def _qcode(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported query dtype {t.dtype}")


# ---------------------------------------------------------------- normalise
def l2_normalize(x: torch.Tensor, out_dtype: str = "f32") -> torch.Tensor:
    """Row-wise x / sqrt(max(sum x^2, 1e-12)) on the GPU; returns float32 or bfloat16."""
    assert x.is_cuda and x.dtype == torch.float32 and x.dim() == 2
    x = x.contiguous()
    out = torch.empty(x.shape, dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16,
                      device=x.device)
    _check(lib().mips_l2_normalize(_ptr(x), x.shape[0], x.shape[1], DTYPE_CODES[out_dtype],
                                   _ptr(out), _stream(x.device)), "mips_l2_normalize")
    return out


# ------------------------------------------------------------------- corpus
@dataclasses.dataclass
class Corpus:
    """A packed, normalised index in the fragment-tiled layout of include/mips.h."""
    packed: torch.Tensor               # uint8 [mips_corpus_bytes]
    row_scale: Optional[torch.Tensor]  # float32 [mips_scale_count] (fp8 and int8)
    n: int
    d: int
    dtype: str
    model_version: Optional[str] = None  # the item tower that produced the rows

    @property
    def code(self) -> int:
        return DTYPE_CODES[self.dtype]


def corpus_bytes(n: int, d: int, dtype: str) -> int:
    return int(lib().mips_corpus_bytes(n, d, DTYPE_CODES[dtype]))


def empty_corpus(n: int, d: int, dtype: str, device="cuda",
                 model_version: Optional[str] = None) -> Corpus:
    nbytes = corpus_bytes(n, d, dtype)
    if nbytes < 0:
        raise MipsError(2, "mips_corpus_bytes")
    packed = torch.empty(nbytes, dtype=torch.uint8, device=device)
    scale = None
    if dtype in SCALED:
        scale = torch.empty(int(lib().mips_scale_count(n)), dtype=torch.float32, device=device)
    return Corpus(packed, scale, n, d, dtype, model_version)


def prepare_rows(corpus: Corpus, x: torch.Tensor, row_offset: int) -> None:
    """Normalise raw rows x (float32 [rows, d], device) and pack them at row_offset."""
    assert x.is_cuda and x.dtype == torch.float32 and x.dim() == 2 and x.shape[1] == corpus.d
    x = x.contiguous()
    _check(lib().mips_prepare_corpus(_ptr(x), x.shape[0], row_offset, corpus.d, corpus.code,
                                     _ptr(corpus.packed), _ptr(corpus.row_scale),
                                     _stream(x.device)), "mips_prepare_corpus")


def prepare_corpus(x: torch.Tensor, dtype: str, model_version: Optional[str] = None) -> Corpus:
    """Normalise and pack a whole raw corpus (float32 [n, d] on the GPU)."""
    c = empty_corpus(x.shape[0], x.shape[1], dtype, x.device, model_version)
    prepare_rows(c, x, 0)
    return c


# -------------------------------------------------------------------- top-k
def workspace_size(b: int, n: int, d: int, k: int, query_dtype: str, corpus_dtype: str,
                   candidates_per_query: Optional[int] = None) -> int:
    """Workspace bytes of mips_topk: the default candidate capacity, or at least
    `candidates_per_query` candidates per query."""
    qc, cc = DTYPE_CODES[query_dtype], DTYPE_CODES[corpus_dtype]
    if candidates_per_query is None:
        return int(lib().mips_topk_workspace_size(b, n, d, k, qc, cc))
    return int(lib().mips_topk_workspace_size_for(b, n, d, k, qc, cc, candidates_per_query))


def masks_workspace_size(b: int, n: int, d: int, k: int, query_dtype: str, corpus_dtype: str,
                         nmasks: int, candidates_per_list: Optional[int] = None) -> int:
    """Workspace bytes of mips_topk_masks: the default candidate capacity per (mask, query)
    list, or at least `candidates_per_list`."""
    qc, cc = DTYPE_CODES[query_dtype], DTYPE_CODES[corpus_dtype]
    return int(lib().mips_topk_masks_workspace_size(b, n, d, k, qc, cc, nmasks,
                                                    candidates_per_list or 0))


def empty_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    # torch's caching allocator returns at least 512-byte aligned blocks
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def check_version(corpus: Corpus, model_version: Optional[str]) -> None:
    """Fails closed: once either side names a model version, both must name the same."""
    if (model_version is not None or corpus.model_version is not None) and \
            model_version != corpus.model_version:
        raise VersionSkew(f"index built by model {corpus.model_version!r}, "
                          f"queries from model {model_version!r}")


def _exclude_arg(exclude: Optional[torch.Tensor], corpus: Corpus, b: int):
    """(contiguous bitmap or None, words per query row): a 1-D bitmap [>= ceil(n/32)] is
    shared by the batch (0 words per row); a 2-D one [b, w >= ceil(n/32)] holds one row per
    query."""
    if exclude is None:
        return None, 0
    words = (corpus.n + 31) // 32
    if not exclude.is_cuda or exclude.dtype not in (torch.int32, torch.uint32):
        raise ValueError("exclude must be an int32/uint32 tensor on the GPU")
    if exclude.dim() == 1:
        if exclude.numel() < words:
            raise ValueError(f"exclude holds {exclude.numel()} words, the corpus needs {words}")
        return exclude.contiguous(), 0
    if exclude.dim() != 2 or exclude.shape[0] != b or exclude.shape[1] < words:
        raise ValueError(f"a per-query exclude must be [{b}, >= {words}], got {tuple(exclude.shape)}")
    return exclude.contiguous(), int(exclude.shape[1])


def topk(queries: torch.Tensor, corpus: Corpus, k: int, exclude: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None,
         out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
         model_version: Optional[str] = None
         ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k by inner product: (scores float32 [b, k], ids int32 [b, k]).

    queries: float32 or bfloat16 [b, d] on the GPU, L2-normalised.
    exclude: optional int32/uint32 bitmap on the GPU, bit i set => id i is never returned:
    [ceil(n/32)] shared by the batch, or [b, w >= ceil(n/32)] with one row per query (a
    per-user set, such as the history that hard-negative mining removes from each user's
    top-k: "Two-Tower Retrieval at Industrial Scale", section "When hard is too hard").
    model_version: the user tower that produced the queries; see check_version.
    """
    check_version(corpus, model_version)
    assert queries.is_cuda and queries.dim() == 2 and queries.shape[1] == corpus.d
    queries = queries.contiguous()
    b = queries.shape[0]
    qc = _qcode(queries)
    if workspace is None:
        nbytes = lib().mips_topk_workspace_size(b, corpus.n, corpus.d, k, qc, corpus.code)
        if nbytes == 0:
            raise MipsError(2, "mips_topk_workspace_size")
        workspace = empty_workspace(nbytes, queries.device)
    if out is None:
        scores = torch.empty((b, k), dtype=torch.float32, device=queries.device)
        ids = torch.empty((b, k), dtype=torch.int32, device=queries.device)
    else:
        scores, ids = out
    exclude, row_words = _exclude_arg(exclude, corpus, b)
    _check(lib().mips_topk(_ptr(queries), qc, b, _ptr(corpus.packed), _ptr(corpus.row_scale),
                           corpus.code, corpus.n, corpus.d, _ptr(exclude), row_words, k,
                           _ptr(scores),
                           _ptr(ids), _ptr(workspace), workspace.numel(),
                           _stream(queries.device)), "mips_topk")
    return scores, ids


def topk_noalloc(queries: torch.Tensor, corpus: Corpus, k: int,
                 exclude: Optional[torch.Tensor] = None,
                 out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                 model_version: Optional[str] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """As topk, through mips_topk_noalloc: the library's own device scratch instead of a
    workspace (nothing is allocated when `out` is given). Calls that overlap on one device
    race; order them on one stream."""
    check_version(corpus, model_version)
    assert queries.is_cuda and queries.dim() == 2 and queries.shape[1] == corpus.d
    queries = queries.contiguous()
    b = queries.shape[0]
    if out is None:
        scores = torch.empty((b, k), dtype=torch.float32, device=queries.device)
        ids = torch.empty((b, k), dtype=torch.int32, device=queries.device)
    else:
        scores, ids = out
    exclude, row_words = _exclude_arg(exclude, corpus, b)
    _check(lib().mips_topk_noalloc(_ptr(queries), _qcode(queries), b, _ptr(corpus.packed),
                                   _ptr(corpus.row_scale), corpus.code, corpus.n, corpus.d,
                                   _ptr(exclude), row_words, k, _ptr(scores), _ptr(ids),
                                   _stream(queries.device)), "mips_topk_noalloc")
    return scores, ids


NOALLOC_SCRATCH_BYTES = 128 << 20


def topk_ranges(queries: torch.Tensor, corpus: Corpus, ranges, k: int,
                exclude: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                model_version: Optional[str] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k per id range [start, end): (scores float32 [r, b, k], ids int32 [r, b, k]), ids
    absolute. One pass per range over the blocks that hold its rows."""
    check_version(corpus, model_version)
    assert queries.is_cuda and queries.dim() == 2 and queries.shape[1] == corpus.d
    queries = queries.contiguous()
    b = queries.shape[0]
    qc = _qcode(queries)
    flat = [int(v) for rg in ranges for v in rg]
    nr = len(flat) // 2
    rg = (C.c_int64 * len(flat))(*flat)
    if workspace is None:
        nbytes = lib().mips_topk_workspace_size(b, corpus.n, corpus.d, k, qc, corpus.code)
        if nbytes == 0:
            raise MipsError(2, "mips_topk_workspace_size")
        workspace = empty_workspace(nbytes, queries.device)
    scores = torch.empty((nr, b, k), dtype=torch.float32, device=queries.device)
    ids = torch.empty((nr, b, k), dtype=torch.int32, device=queries.device)
    exclude, row_words = _exclude_arg(exclude, corpus, b)
    _check(lib().mips_topk_ranges(_ptr(queries), qc, b, _ptr(corpus.packed),
                                  _ptr(corpus.row_scale), corpus.code, corpus.n, corpus.d,
                                  _ptr(exclude), row_words, C.cast(rg, C.c_void_p), nr, k,
                                  _ptr(scores),
                                  _ptr(ids), _ptr(workspace), workspace.numel(),
                                  _stream(queries.device)), "mips_topk_ranges")
    return scores, ids


def merge_topk(scores: torch.Tensor, ids: torch.Tensor, offsets, k: int
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge p sorted result lists per query (scores float32 / ids int32 [p, b, k_in] on the
    GPU, list l's ids shifted by offsets[l]) into one top-k: (scores [b, k], ids [b, k])."""
    assert scores.is_cuda and scores.dtype == torch.float32 and scores.dim() == 3
    assert ids.shape == scores.shape and ids.dtype == torch.int32 and ids.device == scores.device
    p, b, k_in = scores.shape
    offs = (C.c_int64 * p)(*[int(o) for o in offsets])
    scores, ids = scores.contiguous(), ids.contiguous()
    out_s = torch.empty((b, k), dtype=torch.float32, device=scores.device)
    out_i = torch.empty((b, k), dtype=torch.int32, device=scores.device)
    _check(lib().mips_merge_topk(_ptr(scores), _ptr(ids), C.cast(offs, C.c_void_p), p, b, k_in, k,
                                 _ptr(out_s), _ptr(out_i), _stream(scores.device)),
           "mips_merge_topk")
    return out_s, out_i


def search_shards(queries: torch.Tensor, shards, k: int, offsets=None,
                  excludes=None, model_version: Optional[str] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k over several indexes (a base index and a fresh shard, or the row shards of one
    corpus): each is searched on its own and the lists are merged. offsets[l] is the id of
    shard l's first row (default: the shards' row counts, cumulated). Every shard must carry
    the queries' model version (check_version), checked before any work is enqueued."""
    for c in shards:
        check_version(c, model_version)
    if offsets is None:
        offsets, o = [], 0
        for c in shards:
            offsets.append(o)
            o += c.n
    lists = [topk(queries, c, k, None if excludes is None else excludes[l],
                  model_version=model_version) for l, c in enumerate(shards)]
    s = torch.stack([t[0] for t in lists])
    i = torch.stack([t[1] for t in lists])
    return merge_topk(s, i, offsets, k)


def topk_multi_interest(queries: torch.Tensor, corpus: Corpus, k: int,
                        exclude: Optional[torch.Tensor] = None,
                        k_per_vector: Optional[int] = None,
                        model_version: Optional[str] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k of users with m interest vectors each (queries [b, m, d], L2-normalised rows):
    an item scores its best match over the user's vectors. Each vector is searched for
    k_per_vector results (default k: exact), then each user's lists are merged."""
    assert queries.dim() == 3
    b, m, d = queries.shape
    kv = k if k_per_vector is None else k_per_vector
    if exclude is not None and exclude.dim() == 2:  # one row per user: one per vector
        exclude = exclude.repeat_interleave(m, dim=0)
    s, i = topk(queries.reshape(b * m, d), corpus, kv, exclude, model_version=model_version)
    out_s = torch.empty((b, k), dtype=torch.float32, device=queries.device)
    out_i = torch.empty((b, k), dtype=torch.int32, device=queries.device)
    _check(lib().mips_merge_interests(_ptr(s), _ptr(i), b, m, kv, k, _ptr(out_s), _ptr(out_i),
                                      _stream(queries.device)), "mips_merge_interests")
    return out_s, out_i


def topk_masks(queries: torch.Tensor, corpus: Corpus, masks: torch.Tensor, k: int,
               workspace: Optional[torch.Tensor] = None, model_version: Optional[str] = None
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Several result sets from one pass over the corpus: masks int32/uint32 [t, w] on the
    GPU (1 <= t <= MAX_MASKS, w >= ceil(n/32)), bit i of row r set => id i is not in result
    set r. Returns (scores float32 [t, b, k], ids int32 [t, b, k])."""
    check_version(corpus, model_version)
    assert queries.is_cuda and queries.dim() == 2 and queries.shape[1] == corpus.d
    words = (corpus.n + 31) // 32
    if not masks.is_cuda or masks.dtype not in (torch.int32, torch.uint32) or masks.dim() != 2:
        raise ValueError("masks must be a 2-D int32/uint32 tensor on the GPU")
    nm = masks.shape[0]
    if not 1 <= nm <= MAX_MASKS or masks.shape[1] < words:
        raise ValueError(f"masks must be [1..{MAX_MASKS}, >= {words}], got {tuple(masks.shape)}")
    queries, masks = queries.contiguous(), masks.contiguous()
    b = queries.shape[0]
    qc = _qcode(queries)
    if workspace is None:
        nbytes = lib().mips_topk_masks_workspace_size(b, corpus.n, corpus.d, k, qc, corpus.code, nm, 0)
        if nbytes == 0:
            raise MipsError(2, "mips_topk_masks_workspace_size")
        workspace = empty_workspace(nbytes, queries.device)
    scores = torch.empty((nm, b, k), dtype=torch.float32, device=queries.device)
    ids = torch.empty((nm, b, k), dtype=torch.int32, device=queries.device)
    _check(lib().mips_topk_masks(_ptr(queries), qc, b, _ptr(corpus.packed), _ptr(corpus.row_scale),
                                 corpus.code, corpus.n, corpus.d, _ptr(masks), nm, masks.shape[1],
                                 k, _ptr(scores), _ptr(ids), _ptr(workspace), workspace.numel(),
                                 _stream(queries.device)), "mips_topk_masks")
    return scores, ids


def topk_types(queries: torch.Tensor, corpus: Corpus, item_types: torch.Tensor, targets, k: int,
               exclude: Optional[torch.Tensor] = None, return_validity: bool = False,
               model_version: Optional[str] = None):
    """One top-k per target item type: a tuple with, per target, (ids [b, k], scores [b, k])
    or (ids, scores, validity) with return_validity. Items of other types are never returned,
    so validity is ids >= 0 (padding marks a type with fewer than k eligible items). Up to
    MAX_MASKS types share one pass over the corpus (mips_topk_masks)."""
    check_version(corpus, model_version)
    assert item_types.is_cuda and item_types.dtype == torch.int32 and item_types.numel() == corpus.n
    words = (corpus.n + 31) // 32
    exclude, _ = _exclude_arg(exclude, corpus, queries.shape[0])
    if exclude is not None and exclude.dim() != 1:
        raise ValueError("topk_types takes one exclusion bitmap for the batch")
    targets = [int(t) for t in targets]
    results = []
    for g0 in range(0, len(targets), MAX_MASKS):
        group = targets[g0:g0 + MAX_MASKS]
        bms = torch.empty((len(group), words), dtype=torch.int32, device=item_types.device)
        for r, t in enumerate(group):
            _check(lib().mips_type_bitmap(_ptr(item_types.contiguous()), corpus.n, t,
                                          _ptr(exclude), _ptr(bms[r]), _stream(item_types.device)),
                   "mips_type_bitmap")
        s, i = topk_masks(queries, corpus, bms, k, model_version=model_version)
        for r in range(len(group)):
            results.append((i[r], s[r], i[r] >= 0) if return_validity else (i[r], s[r]))
    return tuple(results)


def recall_at_k(approx_ids, exact_ids) -> "np.ndarray":
    """Per query, the fraction of the exact result's ids (padding -1 ignored) that the
    approximate result contains, in any order."""
    import numpy as np
    a = np.asarray(approx_ids)
    e = np.asarray(exact_ids)
    out = np.empty(e.shape[0])
    for q in range(e.shape[0]):
        want = e[q][e[q] >= 0]
        out[q] = 1.0 if want.size == 0 else np.isin(want, a[q][a[q] >= 0]).mean()
    return out


def recall_vs_exact(approx_ids, queries: torch.Tensor, corpus: Corpus, k: int,
                    exclude: Optional[torch.Tensor] = None,
                    model_version: Optional[str] = None) -> "np.ndarray":
    """Recall@k of an approximate index's ids [b, >= k] against this library's exact top-k
    of the same queries: measures the index apart from the model (exact neighbours by brute
    force on a query sample, then the fraction an ANN structure returns; "Two-Tower Retrieval
    at Industrial Scale", section on evaluation)."""
    _, ids = topk(queries, corpus, k, exclude, model_version=model_version)
    return recall_at_k(approx_ids, ids.cpu().numpy())


def set_timing_events(before, after) -> None:
    """Record hipEvents around the main score kernel of later topk calls (None, None stops)."""
    lib().mips_set_timing_events(before, after)
