"""GPU parity of the HIP path against the CPU oracle (small and ragged shapes, edge cases,
invariants). Every call goes through the C ABI of libmips.so."""
import numpy as np
import pytest
import torch

import exact_inner_product_amd as mips
import oracle
from tests.mips_check import (TOL, check_topk, floor_for, int8_step, ref_scores, ref_topk,
                               untile)
from workloads import Workload, bitmap_from_ids

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def _workload(n, d, b, k, cdt, qdt, seed, excl=0.0):
    return Workload("case", "clustered", n=n, d=d, b=b, k=k, corpus_dtype=cdt, query_dtype=qdt,
                    clusters=max(2, n // 40), exclude_frac=excl, seed=seed)


def _gpu_inputs(w, x, qraw, dev):
    corpus = mips.prepare_corpus(torch.from_numpy(x).to(dev), w.corpus_dtype)
    q = mips.l2_normalize(torch.from_numpy(qraw).to(dev), w.query_dtype)
    return corpus, q


def _excl_tensor(bitmap, dev):
    if bitmap is None:
        return None
    return torch.from_numpy(bitmap.view(np.int32)).to(dev)


def run_case(n, d, b, k, cdt, qdt, seed, excl=0.0, workspace_bytes=None, x=None, qraw=None,
             bitmap=None):
    dev = _dev()
    w = _workload(n, d, b, k, cdt, qdt, seed, excl)
    x = w.corpus() if x is None else x
    qraw = w.queries() if qraw is None else qraw
    excluded = None
    if bitmap is None:
        bitmap = w.exclude_bitmap()
        if bitmap is not None:
            excluded = set(w.excluded_ids().tolist())
    else:
        ids = np.arange(n)
        excluded = set(ids[((bitmap[ids >> 5] >> (ids & 31).astype(np.uint32)) & 1) == 1].tolist())
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    if workspace_bytes is None:
        workspace_bytes = mips.workspace_size(b, n, d, k, qdt, cdt)
    ws = mips.empty_workspace(workspace_bytes, dev)
    print(f"case n={n} d={d} b={b} k={k} {cdt}/{qdt} excl={excl} seed={seed}", flush=True)
    s, i = mips.topk(q, corpus, k, _excl_tensor(bitmap, dev), workspace=ws)
    torch.cuda.synchronize()
    s, i = s.cpu().numpy(), i.cpu().numpy()
    c_or, sc_or = oracle.prepare(x, cdt)
    q_or, _ = oracle.prepare(qraw, qdt)
    o_s, o_i = ref_topk(q_or, qdt, c_or, cdt, k, row_scale=sc_or, exclude=bitmap)
    st = check_topk(s, i, o_s, o_i, q_or, qdt, c_or, cdt, sc_or, excluded or set(), n, TOL[cdt],
                    floor=floor_for(cdt, qdt))
    st.update(_ws_counts(ws))
    print(f"case stats: {st}", flush=True)
    return st


def _ws_counts(ws):
    """The diagnostic counts a call leaves in bytes 0..7 of its workspace (include/mips.h):
    lists queued for the rescue pass, lists resolved by the exact rescan."""
    c = ws[:8].cpu().numpy().view(np.uint32)
    return {"queued": int(c[0]), "rescans": int(c[1])}


# --------------------------------------------------------------- prepare parity
@pytest.mark.parametrize("dtype,d", [("f32", 16), ("f32", 64), ("f32", 128), ("bf16", 16),
                                     ("bf16", 32), ("bf16", 64), ("bf16", 128), ("bf16", 256),
                                     ("fp8", 64), ("fp8", 128), ("fp8", 256), ("int8", 32),
                                     ("int8", 64), ("int8", 128), ("int8", 256)])
def test_prepare_matches_oracle_codes(dtype, d):
    dev = _dev()
    rng = np.random.default_rng(d)
    n = 1000 + 17
    x = (rng.standard_normal((n, d)) * rng.uniform(0.01, 30, (n, 1))).astype(np.float32)
    x[5] = 0.0                         # zero row stays zero (scale 1 for fp8)
    corpus = mips.prepare_corpus(torch.from_numpy(x).to(dev), dtype)
    torch.cuda.synchronize()
    got = untile(corpus.packed.cpu().numpy(), n, d, dtype)
    want, scale = oracle.prepare(x, dtype)
    y = oracle.normalize(x)
    if dtype == "f32":
        # both sides normalise in binary32, in different summation orders: each is within
        # (d/2 + 3) 2^-24 of the exact row (a d-term sum, a square root, a quotient)
        bound = (d / 2 + 3) * 2.0 ** -24 * np.abs(y)
        assert np.all(np.abs(got.astype(np.float64) - y) <= bound)
        assert np.all(np.abs(want.astype(np.float64) - y) <= bound)
        return
    gs = None
    if dtype == "fp8":
        gs = corpus.row_scale.cpu().numpy()[:n]
        same = gs == scale
        # a scale may differ only where max|y| sits within fp32 rounding of 448 * 2^t
        amax = np.abs(y).max(axis=1)
        edge = np.abs(amax / (448 * np.minimum(gs, scale)) - 1) < 1e-6
        assert np.all(same | edge)
        assert gs[5] == 1.0
        assert np.all(corpus.row_scale.cpu().numpy()[n:] == 1.0)   # padding rows
    if dtype == "int8":
        gs = corpus.row_scale.cpu().numpy()[:n]
        # scale = max|y| / 127 in fp32 on the GPU, from the fp64 row in the oracle
        assert np.all(np.abs(gs / scale - 1) <= 1e-6)
        assert gs[5] == np.float32(1e-12)
        # every code within one step; the reconstruction within half a step (plus the
        # difference of the two scales)
        assert np.all(np.abs(got.astype(np.int32) - want.astype(np.int32)) <= 1)
        assert np.mean(got == want) > 0.999
        gv = oracle.decode(got, dtype, gs)
        assert np.all(np.abs(gv - y) <= gs[:, None] * (0.5 + 1e-4) + 1e-7)
        return
    gv = oracle.decode(got, dtype, gs)
    ov = oracle.decode(want, dtype, scale)
    exact = np.mean(got == want)
    assert exact > 0.999, f"only {exact:.5f} of the codes match"
    # every mismatch is one code step at most: |difference| <= one ulp of the larger value
    ulp_bits = 7 if dtype == "bf16" else 3
    diff = np.abs(gv - ov)
    bound = np.maximum(np.abs(gv), np.abs(ov)) * 2.0 ** -ulp_bits + (2.0 ** -9) * (1 if gs is None else np.maximum(gs, scale)[:, None])
    assert np.all(diff <= bound)
    assert np.all(got[5] == 0)


@pytest.mark.parametrize("dtype,d", [("f32", 16), ("f32", 128), ("bf16", 64), ("bf16", 256),
                                     ("fp8", 128), ("int8", 32), ("int8", 256)])
def test_prepare_unaligned_source_matches_aligned(dtype, d):
    """A source that is 4- but not 16-byte aligned is read with 4-byte loads instead of
    16-byte ones; the packed bytes and row scales are the same, bit for bit. Two chunks with
    a row offset, the second ragged."""
    dev = _dev()
    rng = np.random.default_rng(100 + d)
    n = 32 * 37 + 11
    x = (rng.standard_normal((n, d)) * rng.uniform(0.01, 30, (n, 1))).astype(np.float32)
    x[3] = 0.0
    flat = torch.empty(n * d + 1, dtype=torch.float32, device=dev)
    flat[1:] = torch.from_numpy(x.ravel()).to(dev)
    shifted = flat[1:].view(n, d)
    assert shifted.data_ptr() % 16 == 4
    aligned = torch.from_numpy(x).to(dev)
    assert aligned.data_ptr() % 16 == 0
    print(f"prepare unaligned {dtype} d={d} n={n}", flush=True)
    out = []
    for src in (aligned, shifted):
        c = mips.empty_corpus(n, d, dtype, dev)
        mips.prepare_rows(c, src[:32 * 20], 0)
        mips.prepare_rows(c, src[32 * 20:], 32 * 20)
        out.append(c)
    torch.cuda.synchronize()
    assert torch.equal(out[0].packed, out[1].packed)
    if out[0].row_scale is not None:
        assert torch.equal(out[0].row_scale.view(torch.int32), out[1].row_scale.view(torch.int32))


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_l2_normalize_matches_oracle(out):
    dev = _dev()
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((333, 100)) * rng.uniform(1e-3, 1e3, (333, 1))).astype(np.float32)
    x[0] = 0.0
    x[1] = 1e-8
    y = mips.l2_normalize(torch.from_numpy(x).to(dev), out)
    torch.cuda.synchronize()
    ref = oracle.normalize(x)
    if out == "f32":
        got = y.cpu().numpy().astype(np.float64)
        assert np.allclose(got, ref, rtol=4e-7, atol=1e-30)
    else:
        got = y.view(torch.int16).cpu().numpy().view(np.uint16)
        want, _ = oracle.prepare(x, "bf16")
        assert np.mean(got == want) > 0.999
        gv, ov = oracle.decode(got, "bf16"), oracle.decode(want, "bf16")
        assert np.all(np.abs(gv - ov) <= np.abs(ov) * 2 ** -7 + 1e-30)
    assert np.all(y.float().cpu().numpy()[0] == 0)


# ----------------------------------------------------------------- top-k parity
DTYPES = [("f32", "f32", 16), ("f32", "f32", 64), ("bf16", "bf16", 128), ("bf16", "bf16", 64),
          ("bf16", "f32", 32), ("bf16", "bf16", 256), ("fp8", "bf16", 256), ("fp8", "bf16", 64),
          ("fp8", "f32", 128), ("int8", "bf16", 128), ("int8", "f32", 64), ("int8", "bf16", 256),
          ("int8", "bf16", 32)]
SHAPES = [(1, 1, 1), (63, 5, 10), (64, 33, 64), (65, 3, 100), (1000, 40, 10), (9000, 7, 1024),
          (40000, 37, 100)]


@pytest.mark.parametrize("cdt,qdt,d", DTYPES)
@pytest.mark.parametrize("n,b,k", SHAPES)
def test_topk_parity(cdt, qdt, d, n, b, k):
    run_case(n, d, b, k, cdt, qdt, seed=n * 7 + b + d)


@pytest.mark.parametrize("cdt,qdt,d", [("bf16", "bf16", 128), ("fp8", "bf16", 128),
                                       ("f32", "f32", 32), ("int8", "bf16", 128)])
def test_topk_with_exclusion(cdt, qdt, d):
    run_case(70001, d, 45, 300, cdt, qdt, seed=5, excl=0.05)
    run_case(3000, d, 6, 50, cdt, qdt, seed=6, excl=0.5)


def test_large_batch_multiple_query_blocks():
    # 2000 queries do not fit one LDS query block: several blocks share each corpus slice
    run_case(20000, 256, 2000, 20, "fp8", "bf16", seed=8)
    run_case(20000, 64, 1100, 30, "bf16", "bf16", seed=9)


def test_all_excluded_and_k_above_eligible():
    dev = _dev()
    n, d = 500, 64
    w = _workload(n, d, 3, 50, "bf16", "bf16", 10)
    corpus, q = _gpu_inputs(w, w.corpus(), w.queries(), dev)
    allx = torch.full(((n + 31) // 32,), -1, dtype=torch.int32, device=dev)
    s, i = mips.topk(q, corpus, 50, allx)
    torch.cuda.synchronize()
    assert torch.all(i == -1) and torch.all(torch.isneginf(s))
    keep = np.array([3, 77, 499])
    bm = np.full((n + 31) // 32, 0xFFFFFFFF, np.uint32)
    for t in keep:
        bm[t >> 5] &= ~np.uint32(1 << (t & 31))
    s, i = mips.topk(q, corpus, 50, torch.from_numpy(bm.view(np.int32)).to(dev))
    torch.cuda.synchronize()
    i = i.cpu().numpy()
    assert np.all(np.sort(i[:, :3], axis=1) == keep) and np.all(i[:, 3:] == -1)


@pytest.mark.parametrize("n", [2000, 50000, 2_000_000])
def test_all_equal_corpus_ties(n):
    """Every score ties: the result is ids 0..k-1 (and, with exclusions, the k smallest
    eligible ids). From n=50000 every item passes the sampled threshold and the candidate
    lists overflow; the rescue's composite threshold (the k-th stored candidate's score and
    id) admits only the tied rows up to that id, so no list reaches the exact rescan."""
    dev = _dev()
    d, k, b = 64, 37, 3
    x = np.ones((n, d), np.float32)
    corpus = mips.prepare_corpus(torch.from_numpy(x).to(dev), "bf16")
    q = mips.l2_normalize(torch.ones((b, d), device=dev), "bf16")
    ws = mips.empty_workspace(mips.workspace_size(b, n, d, k, "bf16", "bf16"), dev)
    s, i = mips.topk(q, corpus, k, workspace=ws)
    torch.cuda.synchronize()
    assert np.all(i.cpu().numpy() == np.arange(k))
    assert torch.all(s == s[0, 0])
    cnt = _ws_counts(ws)
    print(f"all equal n={n}: {cnt}", flush=True)
    assert cnt["rescans"] == 0
    if n >= 50000:
        assert cnt["queued"] == b
    excl = np.array([0, 1, 5, 31, 32, 36])
    bm = bitmap_from_ids(excl, n)
    s, i = mips.topk(q, corpus, k, torch.from_numpy(bm.view(np.int32)).to(dev))
    torch.cuda.synchronize()
    want = [t for t in range(n) if t not in set(excl.tolist())][:k]
    assert np.all(i.cpu().numpy() == np.array(want))


def test_small_workspace_is_still_exact():
    """A workspace with room for one candidate per query and list segment: the lists
    overflow, every query is rescued (and rescanned exactly where the rescue's room of one
    candidate per segment overflows too), and the result still matches the oracle."""
    n, d, b, k = 30000, 128, 9, 40
    wsb = mips.workspace_size(b, n, d, k, "bf16", "bf16", candidates_per_query=1)
    st = run_case(n, d, b, k, "bf16", "bf16", seed=12, workspace_bytes=wsb)
    assert st["queued"] == b


def _sampled_blocks(n, k, g_max=8192):
    """Blocks the sample pass reads: an even integer stride over the 32-row blocks, G of them
    (a 16th of the blocks but no more than ceil(6 n32 / k), enough for about 6 of the k best
    items; at least 4 k, at most 8192)."""
    n32 = (n + 31) // 32
    g = min(n32, g_max, max(min(n32 // 16, (6 * n32 + k - 1) // k), 4 * k))
    step = (n32 << 32) // g
    return np.array([(j * step) >> 32 for j in range(g)], np.int64)


def test_estimate_shortfall_is_rescued():
    """The estimated threshold sits at a low delegate rank. Planting 40 near-duplicates of
    the query, one per sampled block, puts that estimate above all but about 40 items of the
    whole corpus: fewer than K candidates survive the main pass, the query is rescued with
    the proven bound, and the result is still exact."""
    n, d, b, k = 2_000_000, 16, 2, 100
    rng = np.random.default_rng(31)
    x = rng.standard_normal((n, d)).astype(np.float32)
    x[:, 0] *= 0.05  # base items are nearly orthogonal to e_0
    blocks = _sampled_blocks(n, k)
    planted = blocks[:: len(blocks) // 40][:40] * 32
    x[planted] = 0.0
    x[planted, 0] = 1.0
    x[planted, 1:] = 0.02 * rng.standard_normal((40, d - 1)).astype(np.float32)
    qraw = np.zeros((b, d), np.float32)
    qraw[:, 0] = 1.0
    qraw[1, 1] = 0.1
    st = run_case(n, d, b, k, "f32", "f32", seed=31, x=x, qraw=qraw)
    assert st["max_err"] <= 1e-5


def test_no_sampled_bound_takes_exact_scan():
    """Fewer than K eligible sampled blocks: there is no sampled bound, so the rescue pass
    gathers every eligible row (excluded items never returned, the rest padded)."""
    n, d, b, k = 400_000, 64, 3, 100
    keep = np.random.default_rng(32).choice(n, 60, replace=False)
    bm = np.full((n + 31) // 32, 0xFFFFFFFF, np.uint32)
    for t in keep:
        bm[t >> 5] &= ~np.uint32(1 << (t & 31))
    run_case(n, d, b, k, "bf16", "bf16", seed=32, bitmap=bm)


# -------------------------------------------------------------------- invariants
def _scores_ids(q, corpus, k, excl=None):
    s, i = mips.topk(q, corpus, k, excl)
    torch.cuda.synchronize()
    return s.cpu().numpy(), i.cpu().numpy()


def test_determinism_and_batch_invariance():
    dev = _dev()
    w = _workload(60000, 128, 70, 200, "bf16", "bf16", 13, excl=0.05)
    corpus, q = _gpu_inputs(w, w.corpus(), w.queries(), dev)
    ex = _excl_tensor(w.exclude_bitmap(), dev)
    s0, i0 = _scores_ids(q, corpus, w.k, ex)
    for _ in range(5):
        s1, i1 = _scores_ids(q, corpus, w.k, ex)
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32)) and np.array_equal(i0, i1)
    for qi in (0, 31, 32, 69):
        s1, i1 = _scores_ids(q[qi:qi + 1], corpus, w.k, ex)
        assert np.array_equal(s0[qi].view(np.uint32), s1[0].view(np.uint32))
        assert np.array_equal(i0[qi], i1[0])


def test_corpus_permutation_invariance():
    dev = _dev()
    w = _workload(20000, 64, 12, 100, "bf16", "bf16", 14)
    x = w.corpus()
    corpus, q = _gpu_inputs(w, x, w.queries(), dev)
    perm = np.random.default_rng(15).permutation(w.n)
    corpus_p = mips.prepare_corpus(torch.from_numpy(x[perm]).to(dev), "bf16")
    s0, i0 = _scores_ids(q, corpus, w.k)
    s1, i1 = _scores_ids(q, corpus_p, w.k)
    # per-item fp32 scores do not depend on the row position: identical score lists
    assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))
    for qi in range(w.b):
        assert set(perm[i1[qi]].tolist()) == set(i0[qi].tolist()) or s0[qi, -1] == s0[qi, -2]


def test_planted_item_exclusion_shift_and_k_prefix():
    dev = _dev()
    w = _workload(30000, 128, 8, 50, "bf16", "bf16", 16)
    x = w.corpus()
    qraw = w.queries()
    planted = [11, 4095, 29999, 7, 100, 20000, 3, 15000]
    for qi, p in enumerate(planted):
        x[p] = qraw[qi]
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    s, i = _scores_ids(q, corpus, 51)
    assert np.array_equal(i[:, 0], planted)
    s2, i2 = _scores_ids(q, corpus, 50)
    assert np.array_equal(i2, i[:, :50]) and np.array_equal(s2, s[:, :50])
    for qi in range(w.b):
        bm = bitmap_from_ids(np.array([planted[qi]]), w.n)
        s3, i3 = _scores_ids(q[qi:qi + 1], corpus, 50, torch.from_numpy(bm.view(np.int32)).to(dev))
        assert np.array_equal(i3[0], i[qi, 1:51])


# ------------------------------------------------------------------ merging
@pytest.mark.parametrize("cdt,qdt,d", [("bf16", "bf16", 128), ("int8", "bf16", 64)])
def test_row_shards_merged_equal_one_pass(cdt, qdt, d):
    """A corpus split by rows into separately packed shards (cuts not multiples of 32),
    each searched alone and the lists merged: the same ids and bitwise the same scores as
    one pass over the whole corpus, and the oracle's top-k."""
    dev = _dev()
    n, b, k = 50000, 37, 300
    w = _workload(n, d, b, k, cdt, qdt, 41)
    x, qraw = w.corpus(), w.queries()
    cuts = [0, 12345, 30001, 30002, n]
    whole, q = _gpu_inputs(w, x, qraw, dev)
    shards = [mips.prepare_corpus(torch.from_numpy(x[lo:hi]).to(dev), cdt, model_version="m7")
              for lo, hi in zip(cuts[:-1], cuts[1:])]
    s1, i1 = _scores_ids(q, whole, k)
    s2, i2 = mips.search_shards(q, shards, k, model_version="m7")
    torch.cuda.synchronize()
    s2, i2 = s2.cpu().numpy(), i2.cpu().numpy()
    assert np.array_equal(i1, i2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    c_or, sc_or = oracle.prepare(x, cdt)
    q_or, _ = oracle.prepare(qraw, qdt)
    o_s, o_i = ref_topk(q_or, qdt, c_or, cdt, k, row_scale=sc_or)
    check_topk(s2, i2, o_s, o_i, q_or, qdt, c_or, cdt, sc_or, set(), n, TOL[cdt],
               floor=floor_for(cdt, qdt))


def test_fresh_shard_merge_matches_oracle_merge():
    """A base index's top-k and a fresh index's shorter list (padded), merged on the GPU,
    against the oracle's merge of the same lists (exact for its inputs: bitwise)."""
    dev = _dev()
    d, b, k = 64, 20, 200
    wb = _workload(30000, d, b, k, "bf16", "bf16", 42)
    wf = _workload(700, d, b, k, "bf16", "bf16", 43)
    base, q = _gpu_inputs(wb, wb.corpus(), wb.queries(), dev)
    fresh, _ = _gpu_inputs(wf, wf.corpus(), wb.queries(), dev)
    sb, ib = mips.topk(q, base, k)
    sf, i_f = mips.topk(q, fresh, k // 10)
    pad_s = torch.full((b, k), float("-inf"), device=dev)
    pad_i = torch.full((b, k), -1, dtype=torch.int32, device=dev)
    pad_s[:, : k // 10], pad_i[:, : k // 10] = sf, i_f
    ls, li = torch.stack([sb, pad_s]), torch.stack([ib, pad_i])
    for kout in (k, 7, 1024):
        ms, mi = mips.merge_topk(ls, li, [0, wb.n], kout)
        torch.cuda.synchronize()
        os_, oi = oracle.merge_topk(ls.cpu().numpy(), li.cpu().numpy(), [0, wb.n], kout)
        assert np.array_equal(mi.cpu().numpy(), oi)
        assert np.array_equal(ms.cpu().numpy().view(np.uint32), os_.view(np.uint32))


# ------------------------------------------------------------------ id ranges
def _range_bitmap(n, lo, hi, base_bitmap=None):
    """Exclusion bitmap that also masks every id outside [lo, hi): the oracle's reading of
    a range's top-k is the top-k of the non-excluded rows inside the range."""
    ids = np.concatenate([np.arange(0, lo), np.arange(hi, n)])
    bm = bitmap_from_ids(ids, n)
    if base_bitmap is not None:
        bm = bm | base_bitmap
    return bm


@pytest.mark.parametrize("cdt,qdt,d,n", [("bf16", "bf16", 128, 20000), ("int8", "bf16", 64, 20000),
                                         ("bf16", "bf16", 64, 400000)])
def test_topk_ranges_match_masked_oracle(cdt, qdt, d, n):
    dev = _dev()
    b, k = 9, 50
    w = _workload(n, d, b, k, cdt, qdt, 51, excl=0.05)
    x, qraw = w.corpus(), w.queries()
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    bm = w.exclude_bitmap()
    ranges = [(0, n), (5, 37), (33, 1000), (1000, n - 1), (12345, 12346), (64, 96),
              (n // 3, n // 3 + 40), (7, n)]
    s, i = mips.topk_ranges(q, corpus, ranges, k, _excl_tensor(bm, dev))
    torch.cuda.synchronize()
    s, i = s.cpu().numpy(), i.cpu().numpy()
    c_or, sc_or = oracle.prepare(x, cdt)
    q_or, _ = oracle.prepare(qraw, qdt)
    for r, (lo, hi) in enumerate(ranges):
        print(f"range {r}: [{lo}, {hi})", flush=True)
        rbm = _range_bitmap(n, lo, hi, bm)
        o_s, o_i = ref_topk(q_or, qdt, c_or, cdt, k, row_scale=sc_or, exclude=rbm)
        ids = np.arange(n)
        excluded = set(ids[((rbm[ids >> 5] >> (ids & 31).astype(np.uint32)) & 1) == 1].tolist())
        check_topk(s[r], i[r], o_s, o_i, q_or, qdt, c_or, cdt, sc_or, excluded, n, TOL[cdt],
                   floor=floor_for(cdt, qdt))
    # the whole-corpus range is mips_topk itself, bitwise
    s0, i0 = _scores_ids(q, corpus, k, _excl_tensor(bm, dev))
    assert np.array_equal(i0, i[0]) and np.array_equal(s0.view(np.uint32), s[0].view(np.uint32))


# ------------------------------------------------------------ multi-interest
@pytest.mark.parametrize("cdt,m,k", [("bf16", 4, 100), ("int8", 2, 500), ("bf16", 8, 256)])
def test_multi_interest_matches_maxsim_oracle(cdt, m, k):
    """Users with m interest vectors: mips_topk over every vector (k each), then the
    per-user merge keeping each id's best score, against the oracle's top-k by the maximum
    over the user's vectors."""
    dev = _dev()
    n, d, b = 30000, 64, 11
    w = _workload(n, d, b * m, k, cdt, "bf16", 61, excl=0.05)
    x, qraw = w.corpus(), w.queries()
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    bm = w.exclude_bitmap()
    s, i = mips.topk_multi_interest(q.reshape(b, m, d), corpus, k, _excl_tensor(bm, dev))
    torch.cuda.synchronize()
    s, i = s.cpu().numpy(), i.cpu().numpy()
    c_or, sc_or = oracle.prepare(x, cdt)
    q_or, _ = oracle.prepare(qraw, "bf16")
    if cdt == "int8":   # the quantised branch per vector, then the maximum
        o_s, o_i = oracle.maxsim_topk_int8(q_or.reshape(b, m, d), "bf16", c_or, k, sc_or,
                                           exclude=bm)
    else:
        o_s, o_i = oracle.maxsim_topk(q_or.reshape(b, m, d), "bf16", c_or, cdt, k,
                                      row_scale=sc_or, exclude=bm)
    excluded = set(w.excluded_ids().tolist())
    # the acceptance rule per user, with the score of an id its best over the user's vectors
    # (int8: within one code step of the row's quantised score per vector, else TOL)
    for u in range(b):
        gi = i[u][i[u] >= 0]
        assert len(set(gi.tolist())) == gi.size and not (set(gi.tolist()) & excluded)
        assert np.all(s[u][:-1] >= s[u][1:])
        e = np.max([ref_scores(q_or[u * m:(u + 1) * m], "bf16", c_or, cdt,
                               np.full(gi.size, v), gi, row_scale=sc_or) for v in range(m)],
                   axis=0)
        if cdt == "int8":
            tol = np.max([int8_step(q_or[u * m:(u + 1) * m], "bf16", sc_or, v, gi)
                          for v in range(m)], axis=0)
        else:
            tol = np.full(gi.size, TOL[cdt])
        assert np.all(np.abs(s[u][: gi.size] - e) <= tol)
        assert np.abs(s[u] - o_s[u].astype(np.float32)).max() <= 2 * tol.max()
        diff = set(gi.tolist()) ^ set(o_i[u].tolist())
        kth = o_s[u, k - 1]
        for t in diff:
            et = np.max(ref_scores(q_or[u * m:(u + 1) * m], "bf16", c_or, cdt,
                                   np.arange(m), np.full(m, t), row_scale=sc_or))
            assert abs(et - kth) <= 2 * tol.max(), (u, t, et, kth)


def test_recall_harness_against_exact():
    dev = _dev()
    w = _workload(20000, 64, 16, 100, "bf16", "bf16", 71)
    corpus, q = _gpu_inputs(w, w.corpus(), w.queries(), dev)
    _, exact = _scores_ids(q, corpus, 100)
    assert np.all(mips.recall_vs_exact(exact, q, corpus, 100) == 1.0)
    half = exact.copy()
    half[:, 1::2] = -1                                   # an "index" that loses every other hit
    assert np.allclose(mips.recall_vs_exact(half, q, corpus, 100), 0.5)
    assert np.all(mips.recall_vs_exact(exact[:, :10], q, corpus, 100) == 0.1)


def test_topk_per_item_type():
    """One result set per target type, against the oracle's top-k with the other types
    masked (and the base exclusion); validity marks padding only."""
    dev = _dev()
    n, d, b, k = 30000, 128, 7, 200
    w = _workload(n, d, b, k, "bf16", "bf16", 81, excl=0.05)
    x, qraw = w.corpus(), w.queries()
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    bm = w.exclude_bitmap()
    types = np.random.default_rng(82).integers(0, 3, n).astype(np.int32)
    types[:150] = 7                     # a rare type: fewer eligible items than k
    res = mips.topk_types(q, corpus, torch.from_numpy(types).to(dev), [0, 2, 7], k,
                          _excl_tensor(bm, dev), return_validity=True)
    c_or, sc_or = oracle.prepare(x, "bf16")
    q_or, _ = oracle.prepare(qraw, "bf16")
    for t, (i, s, v) in zip([0, 2, 7], res):
        i, s, v = i.cpu().numpy(), s.cpu().numpy(), v.cpu().numpy()
        other = np.nonzero(types != t)[0]
        tbm = bitmap_from_ids(other, n) | bm
        o_s, o_i = ref_topk(q_or, "bf16", c_or, "bf16", k, exclude=tbm)
        excluded = set(other.tolist()) | set(w.excluded_ids().tolist())
        check_topk(s, i, o_s, o_i, q_or, "bf16", c_or, "bf16", None, excluded, n, TOL["bf16"],
                   floor=floor_for("bf16", "bf16"))
        assert np.array_equal(v, i >= 0)
        assert np.all(types[i[i >= 0]] == t)


@pytest.mark.parametrize("cdt,qdt,d,n,b,k", [
    ("bf16", "bf16", 128, 120000, 9, 1024),   # K at its maximum on the sampled path
    ("int8", "bf16", 128, 120000, 9, 1024),
    ("bf16", "bf16", 256, 90000, 300, 64),    # one wave per SIMD, two query blocks
    ("f32", "f32", 128, 70000, 40, 200),      # one wave per SIMD, f32 MFMA
    ("fp8", "f32", 64, 150000, 70, 300),      # two blocks per stage with two waves
])
def test_sampled_path_across_geometries(cdt, qdt, d, n, b, k):
    run_case(n, d, b, k, cdt, qdt, seed=n + d + k, excl=0.05)


# ------------------------------------------------------- one bitmap per query
def _per_query_masks(n, b, rng, o_i=None):
    """[b, words] bitmaps with a different shape per query: random fractions from 0 to 30%,
    one empty row, one row that keeps only 30 ids (fewer than k: padded), and, given the
    oracle's unmasked top ids o_i, rows that remove each query's own best ids (the main pass
    then finds fewer than k eligible candidates above its estimate)."""
    words = (n + 31) // 32
    rows = np.zeros((b, words), np.uint32)
    for qi in range(b):
        kind = qi % 5
        if kind == 0:
            ids = np.empty(0, np.int64)
        elif kind == 1:
            keep = rng.choice(n, 30, replace=False)
            ids = np.setdiff1d(np.arange(n), keep)
        elif kind == 2 and o_i is not None:
            ids = o_i[qi][o_i[qi] >= 0]
        else:
            ids = rng.choice(n, int(n * rng.uniform(0.02, 0.3)), replace=False)
        rows[qi] = bitmap_from_ids(ids, n)
    return rows


def _check_per_query(s, i, rows, q_or, qdt, c_or, cdt, sc_or, n, k):
    ids_all = np.arange(n)
    for qi in range(rows.shape[0]):
        bm = rows[qi]
        o_s, o_i = ref_topk(q_or[qi:qi + 1], qdt, c_or, cdt, k, row_scale=sc_or, exclude=bm)
        excluded = set(ids_all[((bm[ids_all >> 5] >> (ids_all & 31).astype(np.uint32)) & 1) == 1].tolist())
        check_topk(s[qi:qi + 1], i[qi:qi + 1], o_s, o_i, q_or[qi:qi + 1], qdt, c_or, cdt, sc_or,
                   excluded, n, TOL[cdt], floor=floor_for(cdt, qdt))


@pytest.mark.parametrize("cdt,qdt,d,n,b,k", [
    ("bf16", "bf16", 128, 12_000, 10, 100),    # every block sampled: the bound is exact rank k
    ("fp8", "bf16", 256, 400_000, 10, 200),   # a strided sample: estimate above the bound
    ("int8", "bf16", 64, 3_000, 6, 50),       # dense pass
    ("f32", "f32", 64, 20_000, 7, 500),       # dense pass, k above some rows' eligible count
    ("bf16", "f32", 64, 1_000_000, 5, 1000),  # k at its maximum
])
def test_per_query_exclusion_matches_oracle(cdt, qdt, d, n, b, k):
    """One bitmap per query (a per-user history): each row of the result is the oracle's
    top-k of that query with its own bitmap, including rows whose bitmap removes the query's
    own best items and rows left with fewer than k eligible ids."""
    dev = _dev()
    w = _workload(n, d, b, k, cdt, qdt, 71 + d)
    x, qraw = w.corpus(), w.queries()
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    c_or, sc_or = oracle.prepare(x, cdt)
    q_or, _ = oracle.prepare(qraw, qdt)
    _, top = ref_topk(q_or, qdt, c_or, cdt, min(k, 300), row_scale=sc_or)
    rows = _per_query_masks(n, b, np.random.default_rng(71), top)
    print(f"case per-query n={n} d={d} b={b} k={k} {cdt}/{qdt}", flush=True)
    s, i = mips.topk(q, corpus, k, torch.from_numpy(rows.view(np.int32)).to(dev))
    torch.cuda.synchronize()
    _check_per_query(s.cpu().numpy(), i.cpu().numpy(), rows, q_or, qdt, c_or, cdt, sc_or, n, k)


def test_per_query_rows_equal_to_shared_bitmap_match_it():
    """A per-query bitmap whose rows all equal the shared bitmap gives the shared result,
    bitwise (the same scores reach the same selection either way); a row stride wider than
    the corpus needs is honoured."""
    dev = _dev()
    n, d, b, k = 1_000_000, 128, 16, 100
    w = _workload(n, d, b, k, "bf16", "bf16", 72, excl=0.05)
    corpus, q = _gpu_inputs(w, w.corpus(), w.queries(), dev)
    bm = w.exclude_bitmap()
    s0, i0 = _scores_ids(q, corpus, k, _excl_tensor(bm, dev))
    wide = np.full((b, bm.size + 5), 0xFFFFFFFF, np.uint32)  # padding words past the corpus
    wide[:, :bm.size] = bm
    s1, i1 = _scores_ids(q, corpus, k, torch.from_numpy(wide.view(np.int32)).to(dev))
    assert np.array_equal(i0, i1) and np.array_equal(s0.view(np.uint32), s1.view(np.uint32))


def test_per_query_exclusion_with_ranges_and_interests():
    """Per-query bitmaps combine with id ranges (each range's top-k of the query's
    eligible rows inside it) and with multi-interest users (one row per user, shared by
    the user's vectors)."""
    dev = _dev()
    n, d, b, k, m = 40_000, 64, 6, 60, 2
    w = _workload(n, d, b * m, k, "bf16", "bf16", 73)
    x, qraw = w.corpus(), w.queries()
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    c_or, sc_or = oracle.prepare(x, "bf16")
    q_or, _ = oracle.prepare(qraw, "bf16")
    rng = np.random.default_rng(73)
    rows = _per_query_masks(n, b * m, rng)
    ranges = [(0, n), (100, 5000), (n // 2, n)]
    s, i = mips.topk_ranges(q, corpus, ranges, k, torch.from_numpy(rows.view(np.int32)).to(dev))
    torch.cuda.synchronize()
    s, i = s.cpu().numpy(), i.cpu().numpy()
    for r, (lo, hi) in enumerate(ranges):
        print(f"per-query range {r}: [{lo}, {hi})", flush=True)
        rr = np.stack([_range_bitmap(n, lo, hi, rows[qi]) for qi in range(b * m)])
        _check_per_query(s[r], i[r], rr, q_or, "bf16", c_or, "bf16", None, n, k)
    # multi-interest: user u's row applies to each of its m vectors
    urows = rows[::m]
    su, iu = mips.topk_multi_interest(q.reshape(b, m, d), corpus, k,
                                      torch.from_numpy(urows.view(np.int32)).to(dev))
    torch.cuda.synchronize()
    su, iu = su.cpu().numpy(), iu.cpu().numpy()
    for u in range(b):
        o_s, o_i = oracle.maxsim_topk(q_or[u * m:(u + 1) * m].reshape(1, m, d), "bf16", c_or,
                                      "bf16", k, exclude=urows[u])
        gi = iu[u][iu[u] >= 0]
        assert gi.size == (o_i[0] >= 0).sum()
        ex = ((urows[u][gi >> 5] >> (gi & 31).astype(np.uint32)) & 1) == 1
        assert not ex.any(), "an id the user's bitmap excludes was returned"
        assert np.abs(su[u][: gi.size] - o_s[0][: gi.size].astype(np.float32)).max() <= TOL["bf16"]


# ----------------------------------------------------------- multi-mask pass
def _typed_masks(n, rng, base=None):
    """Four exclusion masks over n ids: three disjoint item types (about 60%, 39% and 1% of
    the rows, so the last is rare) and an overlapping mask that keeps a random half; each
    with the optional shared bitmap folded in."""
    types = rng.choice(3, n, p=[0.6, 0.39, 0.01]).astype(np.int32)
    rows = [bitmap_from_ids(np.nonzero(types != t)[0], n) for t in range(3)]
    rows.append(bitmap_from_ids(rng.choice(n, n // 2, replace=False), n))
    rows = np.stack(rows)
    if base is not None:
        rows |= base
    return rows


def _check_mask_rows(s, i, rows, q_or, qdt, c_or, cdt, sc_or, n, k):
    ids_all = np.arange(n)
    for t in range(rows.shape[0]):
        print(f"mask {t}", flush=True)
        bm = rows[t]
        o_s, o_i = ref_topk(q_or, qdt, c_or, cdt, k, row_scale=sc_or, exclude=bm)
        excluded = set(ids_all[((bm[ids_all >> 5] >> (ids_all & 31).astype(np.uint32)) & 1) == 1].tolist())
        check_topk(s[t], i[t], o_s, o_i, q_or, qdt, c_or, cdt, sc_or, excluded, n, TOL[cdt],
                   floor=floor_for(cdt, qdt))


@pytest.mark.parametrize("cdt,qdt,d,n,b,k", [
    ("bf16", "bf16", 128, 300_000, 20, 100),   # a strided sample of blocks
    ("int8", "bf16", 64, 6_000, 9, 50),        # every block sampled
    ("int8", "bf16", 64, 60_000, 9, 50),       # a strided sample
    ("fp8", "bf16", 256, 3_000, 6, 40),        # dense pass
    ("f32", "f32", 32, 20_000, 7, 300),        # dense pass, more queries than one fragment
    ("bf16", "f32", 64, 1_000_000, 5, 1000),   # k at its maximum
    ("bf16", "bf16", 128, 100_000, 200, 64),   # two query blocks of 128
    ("fp8", "bf16", 128, 200_000, 6, 50),      # fp8 scale operands on the sampled path
    ("f32", "f32", 64, 150_000, 5, 30),        # f32 MFMA, sampled
    ("bf16", "bf16", 256, 100_000, 40, 20),    # one wave per SIMD
])
def test_topk_masks_match_oracle(cdt, qdt, d, n, b, k):
    """Several result sets from one pass: each mask's result is the oracle's top-k with that
    mask, and equals mips_topk run with the mask as its exclusion bitmap, bitwise."""
    dev = _dev()
    w = _workload(n, d, b, k, cdt, qdt, 91 + d, excl=0.05)
    x, qraw = w.corpus(), w.queries()
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    rows = _typed_masks(n, np.random.default_rng(91), w.exclude_bitmap())
    print(f"case masks n={n} d={d} b={b} k={k} {cdt}/{qdt}", flush=True)
    s, i = mips.topk_masks(q, corpus, torch.from_numpy(rows.view(np.int32)).to(dev), k)
    torch.cuda.synchronize()
    s, i = s.cpu().numpy(), i.cpu().numpy()
    for t in range(rows.shape[0]):
        s1, i1 = _scores_ids(q, corpus, k, _excl_tensor(rows[t], dev))
        assert np.array_equal(i1, i[t]) and np.array_equal(s1.view(np.uint32), s[t].view(np.uint32)), t
    c_or, sc_or = oracle.prepare(x, cdt)
    q_or, _ = oracle.prepare(qraw, qdt)
    _check_mask_rows(s, i, rows, q_or, qdt, c_or, cdt, sc_or, n, k)


def test_topk_masks_edge_sets_and_rescue():
    """Masks that exclude every row, leave fewer than k rows, or exclude nothing; one to
    three masks per pass; and a workspace of one candidate per list segment, so that every
    list overflows and is rescued: all equal the oracle."""
    dev = _dev()
    n, d, b, k = 200_000, 128, 8, 50
    w = _workload(n, d, b, k, "bf16", "bf16", 92)
    x, qraw = w.corpus(), w.queries()
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    rng = np.random.default_rng(92)
    words = (n + 31) // 32
    keep = rng.choice(n, 20, replace=False)
    rows = np.stack([np.full(words, 0xFFFFFFFF, np.uint32),
                     bitmap_from_ids(np.setdiff1d(np.arange(n), keep), n),
                     np.zeros(words, np.uint32)])
    c_or, sc_or = oracle.prepare(x, "bf16")
    q_or, _ = oracle.prepare(qraw, "bf16")
    for nm in (1, 2, 3):
        s, i = mips.topk_masks(q, corpus, torch.from_numpy(rows[:nm].view(np.int32)).to(dev), k)
        torch.cuda.synchronize()
        print(f"masks {nm}", flush=True)
        _check_mask_rows(s.cpu().numpy(), i.cpu().numpy(), rows[:nm], q_or, "bf16", c_or, "bf16",
                         None, n, k)
    ws = mips.empty_workspace(mips.masks_workspace_size(b, n, d, k, "bf16", "bf16", 3, 1), dev)
    s, i = mips.topk_masks(q, corpus, torch.from_numpy(rows.view(np.int32)).to(dev), k, workspace=ws)
    torch.cuda.synchronize()
    print("masks with one candidate per segment", flush=True)
    _check_mask_rows(s.cpu().numpy(), i.cpu().numpy(), rows, q_or, "bf16", c_or, "bf16", None, n, k)


def test_topk_types_more_than_one_pass():
    """Six target types take two multi-mask passes (four, then two); each result set still
    holds only its type and equals the oracle."""
    dev = _dev()
    n, d, b, k = 50_000, 64, 5, 30
    w = _workload(n, d, b, k, "bf16", "bf16", 93)
    x, qraw = w.corpus(), w.queries()
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    types = np.random.default_rng(93).integers(0, 6, n).astype(np.int32)
    targets = [5, 0, 3, 1, 4, 2]
    res = mips.topk_types(q, corpus, torch.from_numpy(types).to(dev), targets, k)
    c_or, _ = oracle.prepare(x, "bf16")
    q_or, _ = oracle.prepare(qraw, "bf16")
    for t, (i, s) in zip(targets, res):
        i, s = i.cpu().numpy(), s.cpu().numpy()
        other = np.nonzero(types != t)[0]
        o_s, o_i = ref_topk(q_or, "bf16", c_or, "bf16", k, exclude=bitmap_from_ids(other, n))
        check_topk(s, i, o_s, o_i, q_or, "bf16", c_or, "bf16", None, set(other.tolist()), n,
                   TOL["bf16"], floor=floor_for("bf16", "bf16"))


@pytest.mark.parametrize("b", [1, 33])
def test_topk_masks_identical_masks_and_ragged_batches(b):
    """Identical masks give identical result sets, each equal to mips_topk with that mask,
    for one query and for a batch that is not a multiple of 32."""
    dev = _dev()
    n, d, k = 70_000, 128, 7
    w = _workload(n, d, b, k, "bf16", "bf16", 94 + b, excl=0.05)
    corpus, q = _gpu_inputs(w, w.corpus(), w.queries(), dev)
    bm = w.exclude_bitmap()
    rows = np.stack([bm, bm, bm])
    s, i = mips.topk_masks(q, corpus, torch.from_numpy(rows.view(np.int32)).to(dev), k)
    torch.cuda.synchronize()
    s, i = s.cpu().numpy(), i.cpu().numpy()
    s1, i1 = _scores_ids(q, corpus, k, _excl_tensor(bm, dev))
    for t in range(3):
        assert np.array_equal(i[t], i1) and np.array_equal(s[t].view(np.uint32), s1.view(np.uint32)), t


def test_no_estimate_overflow_falls_back_to_exact_rescan():
    """A bitmap that keeps only a contiguous run of 8,000 ids: too few sampled blocks hold
    an eligible row for any estimate or bound, so the list is rescued with a threshold every
    row passes; with room for about 2,048 candidates that rescue overflows, and the exact
    rescan gives the result."""
    n, d, b, k = 400_000, 64, 3, 100
    keep = np.arange(100_000, 108_000)
    bm = bitmap_from_ids(np.setdiff1d(np.arange(n), keep), n)
    ws = mips.workspace_size(b, n, d, k, "bf16", "bf16", candidates_per_query=2048)
    st = run_case(n, d, b, k, "bf16", "bf16", seed=95, bitmap=bm, workspace_bytes=ws)
    assert st["queued"] == b and st["rescans"] == b


def _cluster_sorted(w):
    """The workload's raw rows reordered so that ids follow the clusters (an index whose ids
    are grouped, as in a catalogue sorted by category)."""
    x = w.corpus()
    return np.ascontiguousarray(x[np.argsort(w.cluster_of_id(), kind="stable")])


@pytest.mark.parametrize("cdt,d,k", [("bf16", 128, 100), ("int8", 64, 500), ("bf16", 64, 1000)])
def test_cluster_sorted_ids_need_no_rescan(cdt, d, k):
    """Ids grouped by cluster put a query's candidates in the few corpus slices of its
    cluster, so the per-slice segments of the main pass overflow. The rescue pass keeps one
    contiguous list per rescued query, so it holds them, and no list reaches the exact
    rescan."""
    n, b = 1_000_000, 32
    w = _workload(n, d, b, k, cdt, "bf16", 96).replace(clusters=1024)
    st = run_case(n, d, b, k, cdt, "bf16", seed=96, x=_cluster_sorted(w), qraw=w.queries())
    assert st["queued"] > 0 and st["rescans"] == 0, st


@pytest.mark.parametrize("k", [100, 1000])
def test_duplicated_top_rows_need_no_rescan(k):
    """40,000 rows identical to a query's own direction, spread over an index of 1.2M rows:
    every list of that query overflows its segments with rows tied at the top score. The
    rescue's composite threshold admits only the tied rows up to the k-th stored id, so the
    query needs no exact rescan, and its result is the k smallest duplicated ids (ties go to
    the lower id)."""
    n, d, b = 1_200_000, 64, 4
    w = _workload(n, d, b, k, "bf16", "bf16", 97)
    x, qraw = w.corpus(), w.queries()
    dup = np.sort(np.random.default_rng(97).choice(n, 40_000, replace=False))
    x[dup] = qraw[0]
    st = run_case(n, d, b, k, "bf16", "bf16", seed=97, x=x, qraw=qraw)
    assert st["queued"] >= 1 and st["rescans"] == 0, st
    dev = _dev()
    corpus, q = _gpu_inputs(w, x, qraw, dev)
    _, i = mips.topk(q, corpus, k)
    torch.cuda.synchronize()
    assert np.array_equal(i[0].cpu().numpy(), dup[:k])
