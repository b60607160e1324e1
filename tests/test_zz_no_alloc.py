"""mips_topk_noalloc (the library's own device scratch, no workspace) against mips_topk on
the same inputs: two calls in a row, the second with a smaller input, each bitwise equal
to mips_topk's result. Through the C ABI of libmips.so."""
import numpy as np
import pytest
import torch

import exact_inner_product_amd as mips
from workloads import Workload

pytestmark = pytest.mark.gpu


def _inputs(n, d, b, k, cdt, qdt, seed, excl, dev):
    w = Workload("noalloc", "clustered", n=n, d=d, b=b, k=k, corpus_dtype=cdt, query_dtype=qdt,
                 clusters=max(2, n // 40), exclude_frac=excl, seed=seed)
    corpus = mips.prepare_corpus(torch.from_numpy(w.corpus()).to(dev), cdt)
    q = mips.l2_normalize(torch.from_numpy(w.queries()).to(dev), qdt)
    bm = w.exclude_bitmap()
    ex = None if bm is None else torch.from_numpy(bm.view(np.int32)).to(dev)
    return corpus, q, ex


def test_noalloc_matches_topk_on_two_calls_the_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    dev = torch.device("cuda:0")
    cases = [(400_000, 128, 96, 300, "bf16", "bf16", 5, 0.05),   # sampled pass, rescue-capable
             (30_000, 64, 17, 40, "int8", "bf16", 6, 0.0)]       # smaller: fewer rows, queries, k
    for n, d, b, k, cdt, qdt, seed, excl in cases:
        corpus, q, ex = _inputs(n, d, b, k, cdt, qdt, seed, excl, dev)
        assert mips.workspace_size(b, n, d, k, qdt, cdt) <= mips.NOALLOC_SCRATCH_BYTES
        print(f"noalloc: n={n} d={d} b={b} k={k} {cdt}/{qdt}", flush=True)
        s0, i0 = mips.topk(q, corpus, k, ex)
        out = (torch.full((b, k), 7.0, device=dev), torch.full((b, k), 7, dtype=torch.int32, device=dev))
        s1, i1 = mips.topk_noalloc(q, corpus, k, ex, out=out)
        torch.cuda.synchronize()
        assert s1.data_ptr() == out[0].data_ptr() and i1.data_ptr() == out[1].data_ptr()
        assert torch.equal(i0, i1)
        assert torch.equal(s0.view(torch.int32), s1.view(torch.int32))


def test_noalloc_rejects_a_call_beyond_its_scratch():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    dev = torch.device("cuda:0")
    b, n, d, k = 1024, 2_000_000, 64, 1000
    assert mips.workspace_size(b, n, d, k, "bf16", "bf16") > mips.NOALLOC_SCRATCH_BYTES
    corpus = mips.empty_corpus(n, d, "bf16", dev)
    q = torch.zeros((b, d), dtype=torch.bfloat16, device=dev)
    with pytest.raises(mips.MipsError, match="workspace too small"):
        mips.topk_noalloc(q, corpus, k)
