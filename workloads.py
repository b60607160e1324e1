"""Seeded synthetic inputs for exhaustive inner-product top-K.

This module is the only code shared by the CPU oracle side (tests, bench baseline)
and the HIP side. It holds none of the method's arithmetic: it produces *raw*,
un-normalised fp32 vectors and "already seen" exclusion sets. Normalisation,
packing, scoring and selection live in `oracle/` and in the HIP library, each
written independently.

Workloads (sizes are the five configurations the retrieval hot path is measured on):

* ``tiny_f32`` -- the toy of "Two-tower retrieval" (mhtirogla.ai, section "Code"):
  8 taste groups x 50 items, D=16, B=128 queries, K=10. Item ``i`` belongs to group
  ``i mod 8`` (the toy numbers items ``r*G + g``); an item is the one-hot group
  centroid plus N(0, 0.3^2) noise per dimension; a query is the one-hot centroid of a
  uniformly drawn group plus U(-0.15, 0.15) noise per dimension (the toy's
  ``0.3*(U-0.5)``). Dimensions 8..15 carry only noise.
* clustered/Zipf corpora (all other workloads): C centres ~ N(0, I_D); cluster sizes
  proportional to 1/(c+1) (Zipf 1.0), rounded to sum exactly N by largest remainder;
  item ids are a seeded random permutation of the cluster-sorted order; an item is
  its centre plus N(0, 0.5^2) noise per dimension; a query is a uniformly drawn
  centre plus N(0, 0.5^2) noise.
* optional exclusion: exactly floor(frac * N) ids drawn uniformly without
  replacement, one set shared by the whole query batch (the shared type mask of
  ``RecsysTwoTowerModel.forward`` in recsys_two_tower_model.py).

Every random stream is derived from ``numpy.random.SeedSequence(seed)`` with a fixed
spawn key per purpose (and per chunk for the corpus), so any chunk of any corpus can
be regenerated independently and in any order.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Iterator, Optional, Tuple

import numpy as np

BASE_SEED = 20260721

# Spawn keys of the independent streams.
_K_CENTRES, _K_PERM, _K_NOISE, _K_QUERIES, _K_EXCLUDE = 0, 1, 2, 3, 4

DEFAULT_CHUNK = 1 << 20  # rows per corpus chunk (a multiple of 256)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "groups" (toy) or "clustered"
    n: int               # corpus rows
    d: int               # embedding width
    b: int               # queries per batch
    k: int               # results per query
    corpus_dtype: str    # "f32", "bf16", "fp8" or "int8"
    query_dtype: str     # "f32" or "bf16"
    clusters: int = 8
    exclude_frac: float = 0.0
    item_sigma: float = 0.5
    query_sigma: float = 0.5
    seed: int = BASE_SEED

    # ------------------------------------------------------------------ helpers
    def _rng(self, *key: int) -> np.random.Generator:
        ss = np.random.SeedSequence(self.seed, spawn_key=tuple(int(x) for x in key))
        return np.random.Generator(np.random.PCG64(ss))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def corpus_elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1}[self.corpus_dtype]

    # ------------------------------------------------------------ clustered parts
    def centres(self) -> np.ndarray:
        if self.kind == "groups":
            c = np.zeros((self.clusters, self.d), np.float32)
            c[np.arange(self.clusters), np.arange(self.clusters)] = 1.0
            return c
        return self._rng(_K_CENTRES).standard_normal((self.clusters, self.d), dtype=np.float32)

    def cluster_sizes(self) -> np.ndarray:
        """Zipf(1.0) sizes summing exactly to n (largest-remainder rounding)."""
        w = 1.0 / np.arange(1, self.clusters + 1, dtype=np.float64)
        exact = self.n * w / w.sum()
        base = np.floor(exact).astype(np.int64)
        rem = self.n - int(base.sum())
        if rem:
            order = np.lexsort((np.arange(self.clusters), -(exact - base)))
            base[order[:rem]] += 1
        return base

    def cluster_of_id(self) -> np.ndarray:
        """int32[n]: cluster of every item id."""
        if self.kind == "groups":
            return (np.arange(self.n) % self.clusters).astype(np.int32)
        sizes = self.cluster_sizes()
        sorted_cluster = np.repeat(np.arange(self.clusters, dtype=np.int32), sizes)
        perm = self._rng(_K_PERM).permutation(self.n)
        out = np.empty(self.n, np.int32)
        out[perm] = sorted_cluster
        return out

    # ------------------------------------------------------------------- corpus
    def corpus_chunk(self, row0: int, rows: int, centres=None, cluster_of_id=None,
                     chunk: int = DEFAULT_CHUNK) -> np.ndarray:
        """Raw fp32 rows [row0, row0+rows). row0 must be a multiple of `chunk`
        unless the request lies inside one chunk."""
        if centres is None:
            centres = self.centres()
        if cluster_of_id is None:
            cluster_of_id = self.cluster_of_id()
        out = np.empty((rows, self.d), np.float32)
        r = row0
        while r < row0 + rows:
            ci = r // chunk
            c0 = ci * chunk
            c1 = min(c0 + chunk, self.n)
            block = self._chunk(ci, c0, c1, centres, cluster_of_id)
            a = r - c0
            e = min(c1, row0 + rows) - c0
            out[r - row0: r - row0 + (e - a)] = block[a:e]
            r = c0 + e
        return out

    def _chunk(self, ci, c0, c1, centres, cluster_of_id) -> np.ndarray:
        rng = self._rng(_K_NOISE, ci)
        rows = c1 - c0
        if self.kind == "groups":
            noise = rng.standard_normal((rows, self.d), dtype=np.float32) * np.float32(0.3)
        else:
            noise = rng.standard_normal((rows, self.d), dtype=np.float32) * np.float32(self.item_sigma)
        noise += centres[cluster_of_id[c0:c1]]
        return noise

    def corpus_chunks(self, chunk: int = DEFAULT_CHUNK, threads: Optional[int] = None
                      ) -> Iterator[Tuple[int, np.ndarray]]:
        """Yield (row0, raw fp32 [rows, d]) for consecutive chunks, generated in parallel."""
        centres = self.centres()
        cid = self.cluster_of_id()
        nchunks = (self.n + chunk - 1) // chunk
        threads = threads or min(16, max(1, len(os.sched_getaffinity(0))))

        def make(ci):
            c0 = ci * chunk
            return c0, self._chunk(ci, c0, min(c0 + chunk, self.n), centres, cid)

        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            window = []
            nxt = 0
            while nxt < nchunks and len(window) < threads:
                window.append(ex.submit(make, nxt))
                nxt += 1
            while window:
                fut = window.pop(0)
                if nxt < nchunks:
                    window.append(ex.submit(make, nxt))
                    nxt += 1
                yield fut.result()

    def corpus(self) -> np.ndarray:
        """Whole raw corpus (only for small workloads)."""
        out = np.empty((self.n, self.d), np.float32)
        for r0, blk in self.corpus_chunks():
            out[r0:r0 + blk.shape[0]] = blk
        return out

    # ------------------------------------------------------------------ queries
    def query_clusters(self) -> np.ndarray:
        return self._rng(_K_QUERIES).integers(0, self.clusters, self.b)

    def queries(self) -> np.ndarray:
        """Raw fp32 queries [b, d]."""
        rng = self._rng(_K_QUERIES)
        g = rng.integers(0, self.clusters, self.b)
        cen = self.centres()
        if self.kind == "groups":
            noise = rng.uniform(-0.15, 0.15, (self.b, self.d)).astype(np.float32)
        else:
            noise = rng.standard_normal((self.b, self.d), dtype=np.float32) * np.float32(self.query_sigma)
        return (cen[g] + noise).astype(np.float32)

    # ---------------------------------------------------------------- exclusion
    def excluded_ids(self) -> Optional[np.ndarray]:
        if self.exclude_frac <= 0.0:
            return None
        m = int(np.floor(self.exclude_frac * self.n))
        return np.sort(self._rng(_K_EXCLUDE).choice(self.n, size=m, replace=False))

    def exclude_bitmap(self) -> Optional[np.ndarray]:
        ids = self.excluded_ids()
        if ids is None:
            return None
        return bitmap_from_ids(ids, self.n)


def typed_masks(n: int, base: Optional[np.ndarray] = None, seed: int = 20261203) -> np.ndarray:
    """Four exclusion masks over n ids for a multi-mask search, uint32 [4, ceil(n/32)]: three
    disjoint item types drawn per id with probabilities 0.6, 0.39 and 0.01 (the last a rare
    type), each mask excluding the ids of the other types, and a random half of the ids;
    the optional shared bitmap `base` is folded into every mask."""
    rng = np.random.default_rng(seed)
    types = rng.choice(3, n, p=[0.6, 0.39, 0.01]).astype(np.int8)
    rows = [bitmap_from_ids(np.nonzero(types != t)[0], n) for t in range(3)]
    rows.append(bitmap_from_ids(rng.choice(n, n // 2, replace=False), n))
    rows = np.stack(rows)
    if base is not None:
        rows |= base
    return rows


def lattice_rows(r0: int, r1: int, d: int, device=None):
    """Raw rows r0..r1-1 of a deterministic pattern, float32 [r1 - r0, d]: element (r, j) is
    ((r * 2654435761 + j * 40503 + 12345) >> 7) % 4093 - 2046, divided by 256. Every value
    is exact in float32, so a GPU-side build (`device` given: a torch tensor made there)
    and a numpy build (`device` None) agree bit for bit. For inputs too large to draw on the
    host: rows far apart can be regenerated one by one."""
    if device is None:
        r = np.arange(r0, r1, dtype=np.int64)[:, None]
        j = np.arange(d, dtype=np.int64)[None, :]
        v = ((r * 2654435761 + j * 40503 + 12345) >> 7) % 4093 - 2046
        return (v.astype(np.float32) / np.float32(256.0)).astype(np.float32)
    import torch
    r = torch.arange(r0, r1, dtype=torch.int64, device=device)[:, None]
    j = torch.arange(d, dtype=torch.int64, device=device)[None, :]
    v = torch.bitwise_right_shift(r * 2654435761 + j * 40503 + 12345, 7) % 4093 - 2046
    return v.to(torch.float32) / 256.0


def bitmap_from_ids(ids: np.ndarray, n: int) -> np.ndarray:
    """uint32[ceil(n/32)]; bit (i & 31) of word (i >> 5) set <=> id i excluded."""
    words = np.zeros((n + 31) // 32, np.uint32)
    ids = np.asarray(ids, np.int64)
    np.bitwise_or.at(words, ids >> 5, (np.uint32(1) << (ids & 31).astype(np.uint32)))
    return words


WORKLOADS = {
    "tiny_f32_n400_d16": Workload("tiny_f32_n400_d16", "groups", n=400, d=16, b=128, k=10,
                                  corpus_dtype="f32", query_dtype="f32", clusters=8),
    "bf16_n1m_d128_b16": Workload("bf16_n1m_d128_b16", "clustered", n=1_000_000, d=128, b=16,
                                  k=100, corpus_dtype="bf16", query_dtype="bf16", clusters=1024),
    "bf16_n10m_d128_b256_excl5": Workload("bf16_n10m_d128_b256_excl5", "clustered",
                                          n=10_000_000, d=128, b=256, k=500,
                                          corpus_dtype="bf16", query_dtype="bf16",
                                          clusters=16384, exclude_frac=0.05),
    "bf16_n100m_d64_b1024": Workload("bf16_n100m_d64_b1024", "clustered", n=100_000_000, d=64,
                                     b=1024, k=1000, corpus_dtype="bf16", query_dtype="bf16",
                                     clusters=65536),
    "fp8_n10m_d256_b4096": Workload("fp8_n10m_d256_b4096", "clustered", n=10_000_000, d=256,
                                    b=4096, k=200, corpus_dtype="fp8", query_dtype="bf16",
                                    clusters=16384),
    # the headline shape with the int8 index of the quantised scoring path
    "int8_n10m_d128_b256_excl5": Workload("int8_n10m_d128_b256_excl5", "clustered",
                                          n=10_000_000, d=128, b=256, k=500,
                                          corpus_dtype="int8", query_dtype="bf16",
                                          clusters=16384, exclude_frac=0.05),
}

# Seeds: each workload gets its own base seed so their streams never coincide.
for _i, _name in enumerate(list(WORKLOADS)):
    WORKLOADS[_name] = WORKLOADS[_name].replace(seed=BASE_SEED + _i + 1)

HEADLINE = "bf16_n10m_d128_b256_excl5"
