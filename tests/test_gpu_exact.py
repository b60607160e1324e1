"""GPU parity on the oracle's own operands. The index is packed on the host from the
oracle's codes (tests.mips_check.tile) and the queries are the oracle's codes, so the GPU
searches exactly the inputs the oracle scores:

* int8 index: the oracle's quantised scoring branch (per-query int8 codes, exact integer dot
  products, then the query scale and the row scale in binary32) and the GPU must return
  identical ids and bitwise identical scores;
* bf16, f32 and fp8 indexes: every returned score within the binary32 accumulation bound
  (D + 2) 2^-24 sum_d |q_d c_d| of the exact score of the GPU's operands (for fp8 the query
  is quantised to E4M3 with a power-of-two scale, as the GPU does), ids identical to the
  exact top-k except swaps within that bound of the K-th score.

The shapes span the dense and the sampled modes, several query blocks, ragged corpus and
batch sizes, K from 1 to 1024, and a shared exclusion bitmap. Every call goes through the
C ABI of libmips.so."""
import numpy as np
import pytest
import torch

import exact_inner_product_amd as mips
import oracle
from tests.mips_check import check_operands, query_tensor, upload_corpus
from workloads import Workload

pytestmark = pytest.mark.gpu

CASES = [
    # cdt, qdt, d, n, b, k, exclusion fraction
    ("int8", "bf16", 128, 3_000, 37, 50, 0.0),       # dense pass
    ("int8", "bf16", 128, 200_003, 70, 100, 0.05),   # sampled, three query fragments
    ("int8", "f32", 64, 150_017, 33, 1024, 0.0),
    ("int8", "bf16", 256, 120_000, 9, 10, 0.05),
    ("int8", "bf16", 32, 50_000, 5, 1, 0.0),
    ("bf16", "bf16", 128, 200_003, 70, 100, 0.05),
    ("bf16", "bf16", 64, 3_000, 33, 64, 0.0),        # dense pass
    ("bf16", "f32", 128, 100_000, 20, 200, 0.0),
    ("bf16", "bf16", 256, 90_000, 17, 300, 0.0),
    ("bf16", "bf16", 16, 80_000, 40, 20, 0.0),
    ("bf16", "bf16", 128, 120_000, 300, 1024, 0.0),  # two query blocks, the largest K
    ("f32", "f32", 128, 60_000, 12, 100, 0.0),
    ("f32", "f32", 16, 5_000, 130, 10, 0.0),
    ("fp8", "bf16", 256, 150_000, 65, 200, 0.0),
    ("fp8", "f32", 128, 100_000, 20, 50, 0.05),
    ("fp8", "bf16", 64, 4_000, 8, 30, 0.0),          # dense pass
]


@pytest.mark.parametrize("cdt,qdt,d,n,b,k,excl", CASES)
def test_search_of_oracle_codes(cdt, qdt, d, n, b, k, excl):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    dev = torch.device("cuda:0")
    w = Workload("case", "clustered", n=n, d=d, b=b, k=k, corpus_dtype=cdt, query_dtype=qdt,
                 clusters=max(2, n // 40), exclude_frac=excl, seed=1000 + n % 977 + d)
    codes, scale = oracle.prepare(w.corpus(), cdt)
    q_codes, _ = oracle.prepare(w.queries(), qdt)
    bm = w.exclude_bitmap()
    excluded = set(w.excluded_ids().tolist()) if bm is not None else set()
    print(f"oracle codes: n={n} d={d} b={b} k={k} {cdt}/{qdt} excl={excl}", flush=True)
    corpus = upload_corpus(codes, scale, cdt, dev)
    q = query_tensor(q_codes, qdt, dev)
    ex = None if bm is None else torch.from_numpy(bm.view(np.int32)).to(dev)
    s, i = mips.topk(q, corpus, k, ex)
    torch.cuda.synchronize()
    stats = check_operands(s.cpu().numpy(), i.cpu().numpy(), q_codes, qdt, codes, cdt, scale,
                           excluded, n, exclude_bitmap=bm)
    print(f"oracle codes: {stats}", flush=True)


def _int8_exact(codes, scale, q_codes, qdt, k, dev, tag):
    n = codes.shape[0]
    print(f"int8 {tag}: n={n} d={codes.shape[1]} b={q_codes.shape[0]} k={k}", flush=True)
    corpus = upload_corpus(codes, scale, "int8", dev)
    s, i = mips.topk(query_tensor(q_codes, qdt, dev), corpus, k)
    torch.cuda.synchronize()
    stats = check_operands(s.cpu().numpy(), i.cpu().numpy(), q_codes, qdt, codes, "int8", scale,
                           set(), n)
    print(f"int8 {tag}: {stats}", flush=True)
    return s.cpu().numpy()


def test_int8_scales_far_from_a_unit_row():
    """Row scales that no normalised row has (up to 40 times its largest, and zero) on a
    sampled int8 search: scores far above 1 and exact zeros must still come out bitwise equal
    to the oracle's quantised branch."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    dev = torch.device("cuda:0")
    n, d, b, k = 120_000, 128, 19, 60
    w = Workload("case", "clustered", n=n, d=d, b=b, k=k, corpus_dtype="int8", query_dtype="bf16",
                 clusters=3000, seed=4242)
    codes, scale = oracle.prepare(w.corpus(), "int8")
    q_codes, _ = oracle.prepare(w.queries(), "bf16")
    rng = np.random.default_rng(7)
    scale = scale.copy()
    big = rng.choice(n, n // 10, replace=False)
    scale[big] = (scale[big] * rng.choice([2.0, 5.0, 40.0], big.size)).astype(np.float32)
    scale[32 * 1000:32 * 1001] = np.float32(0.5)        # one whole block far out of range
    scale[rng.choice(n, 200, replace=False)] = np.float32(0.0)
    _int8_exact(codes, scale, q_codes, "bf16", k, dev, "wide scales")


def test_int8_negative_thresholds():
    """Queries opposite to every row: every score and the K-th threshold are negative (the
    fast path's bound then lies on the other side of the products), results still exact."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    dev = torch.device("cuda:0")
    n, d, b, k = 60_000, 64, 7, 100
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((n, d)) * 0.1).astype(np.float32)
    x[:, 0] += 1.0
    qraw = (rng.standard_normal((b, d)) * 0.1).astype(np.float32)
    qraw[:, 0] -= 1.0
    codes, scale = oracle.prepare(x, "int8")
    q_codes, _ = oracle.prepare(qraw, "bf16")
    s = _int8_exact(codes, scale, q_codes, "bf16", k, dev, "negative scores")
    assert (s < 0).all()
