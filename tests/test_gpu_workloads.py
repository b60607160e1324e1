"""Parity at the five measured workload sizes, in the launch configuration the benchmark
times (full batch, default workspace). Large workloads are checked on sampled queries that
the oracle computes one by one; every query is checked for properties that hold at any
size (well-formed, sorted, no excluded id, scores within the unit bound)."""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import exact_inner_product_amd as mips
import oracle
from tests.mips_check import (TOL, check_operands, check_topk, floor_for, operand_reference,
                               operands_are_inputs, query_tensor, ref_topk, threads,
                               upload_corpus)
from workloads import WORKLOADS

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def build_both(w, dev):
    """One pass over the raw chunks feeds both sides: GPU prepare and oracle prepare."""
    corpus = mips.empty_corpus(w.n, w.d, w.corpus_dtype, dev)
    codes = np.empty((w.n, w.d), {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8,
                                  "int8": np.int8}[w.corpus_dtype])
    scale = np.empty(w.n, np.float32) if w.corpus_dtype in ("fp8", "int8") else None

    def cpu(r0, blk):
        c, s = oracle.prepare(blk, w.corpus_dtype)
        codes[r0:r0 + blk.shape[0]] = c
        if scale is not None:
            scale[r0:r0 + blk.shape[0]] = s

    with cf.ThreadPoolExecutor(threads()) as ex:
        pending = []
        for r0, blk in w.corpus_chunks():
            mips.prepare_rows(corpus, torch.from_numpy(blk).to(dev), r0)
            pending.append(ex.submit(cpu, r0, blk))
            if len(pending) >= threads():
                pending.pop(0).result()
        for f in pending:
            f.result()
    qraw = w.queries()
    q = mips.l2_normalize(torch.from_numpy(qraw).to(dev), w.query_dtype)
    q_or, _ = oracle.prepare(qraw, w.query_dtype)
    bm = w.exclude_bitmap()
    torch.cuda.synchronize()
    return corpus, q, bm, codes, scale, q_or


_STATE = {}


def workload_state(name, sample, exact_sample):
    """Builds workload `name` once per test process and runs both GPU searches in the
    launch configuration the benchmark times: each side builds its own index from the raw
    rows (GPU prepare, oracle prepare), and the GPU also searches the oracle's own codes.
    Keeps host copies of what the checks need; frees the device memory."""
    if name in _STATE:
        return _STATE[name]
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    dev = torch.device("cuda:0")
    w = WORKLOADS[name]
    print(f"workload {name}: building inputs", flush=True)
    corpus, q, bm, codes, scale, q_or = build_both(w, dev)
    excl = None if bm is None else torch.from_numpy(bm.view(np.int32)).to(dev)
    print(f"workload {name}: mips_topk b={w.b}", flush=True)
    s, i = mips.topk(q, corpus, w.k, excl)
    torch.cuda.synchronize()
    s, i = s.cpu().numpy(), i.cpu().numpy()
    del corpus, q
    torch.cuda.empty_cache()
    oc = upload_corpus(codes, scale, w.corpus_dtype, dev)
    s2, i2 = mips.topk(query_tensor(q_or, w.query_dtype, dev), oc, w.k, excl)
    torch.cuda.synchronize()
    s2, i2 = s2.cpu().numpy(), i2.cpu().numpy()
    del oc, excl
    torch.cuda.empty_cache()
    st = dict(w=w, s=s, i=i, s2=s2, i2=i2, bm=bm, codes=codes, scale=scale, q_or=q_or,
              excluded=set(w.excluded_ids().tolist()) if bm is not None else set(),
              sel=np.array(sorted(set(sample)), np.int64),
              xsel=np.array(sorted(set(exact_sample)), np.int64))
    _STATE.clear()  # one workload's host arrays at a time
    _STATE[name] = st
    return st


def check_end_to_end(st):
    """Every query: well-formed and within the unit bound; the sampled queries against the
    oracle's top-k of its own index (the tolerance rule of check_topk)."""
    w, s, i, excluded = st["w"], st["s"], st["i"], st["excluded"]
    # relative rounding of a stored unit row: int8 moves each element by at most
    # max|y| / 254, i.e. the row by at most sqrt(D) / 254 (< 2^-4 for D <= 256)
    delta = {"f32": 2 ** -23, "bf16": 2 ** -8, "fp8": 2 ** -4, "int8": 2 ** -4}[w.corpus_dtype]
    kk = min(w.k, w.n - len(excluded))
    assert np.all(i[:, :kk] >= 0) and np.all(i[:, :kk] < w.n)
    assert np.all(s[:, :-1] >= s[:, 1:])
    assert np.all(np.abs(s[:, :kk]) <= (1 + delta) ** 2 + 1e-3)
    if excluded:
        ex = np.array(sorted(excluded))
        assert not np.isin(i, ex).any()
    sel = st["sel"]
    print(f"workload {w.name}: oracle on queries {sel.tolist()}", flush=True)
    o_s, o_i = ref_topk(st["q_or"][sel], w.query_dtype, st["codes"], w.corpus_dtype, w.k,
                        row_scale=st["scale"], exclude=st["bm"], threads=threads())
    stats = check_topk(s[sel], i[sel], o_s, o_i, st["q_or"][sel], w.query_dtype, st["codes"],
                       w.corpus_dtype, st["scale"], excluded, w.n, TOL[w.corpus_dtype],
                       floor=floor_for(w.corpus_dtype, w.query_dtype))
    print(f"workload {w.name}: end to end: {stats}", flush=True)


def check_oracle_codes(st, part=0, parts=1):
    """The search of the oracle's own codes against the exact scores of its operands
    (check_operands), on every parts-th of the exact sample from `part`."""
    w = st["w"]
    xsel = st["xsel"][part::parts]
    print(f"workload {w.name}: oracle on {xsel.size} queries", flush=True)
    ref = operand_reference(st["q_or"][xsel], w.query_dtype, st["codes"], w.corpus_dtype, w.k,
                            row_scale=st["scale"], exclude=st["bm"], threads_=threads())
    stats = check_operands(st["s2"][xsel], st["i2"][xsel], st["q_or"][xsel], w.query_dtype,
                           st["codes"], w.corpus_dtype, st["scale"], st["excluded"], w.n,
                           exclude_bitmap=st["bm"], ref=ref)
    print(f"workload {w.name}: oracle codes, {xsel.size} queries: {stats}", flush=True)


def _spread(b, count, seed):
    """count seeded query indices of a batch of b, the first and the last included."""
    rng = np.random.default_rng(seed)
    return sorted({0, b - 1, *(1 + rng.choice(b - 2, count - 2, replace=False)).tolist()})


# Each test stays well under three minutes (the oracle on at most about 64 queries of
# 10^7 rows, or 16 of 10^8), so a test run reports progress at least that often.
SPECS = {
    "tiny_f32_n400_d16": (range(128), range(128)),
    "bf16_n1m_d128_b16": (range(16), range(16)),
    "bf16_n10m_d128_b256_excl5": ([0, 1, 31, 32, 100, 128, 200, 255], range(256)),
    "fp8_n10m_d256_b4096": ([0, 1, 511, 512, 2047, 3000, 4094, 4095], _spread(4096, 64, 5)),
    "int8_n10m_d128_b256_excl5": ([0, 1, 63, 64, 127, 200, 254, 255], range(256)),
    "bf16_n100m_d64_b1024": ([0, 1023], _spread(1024, 64, 4)),
}
PARTS = {"bf16_n10m_d128_b256_excl5": 4, "int8_n10m_d128_b256_excl5": 4,
         "bf16_n100m_d64_b1024": 4}


def _state(name):
    return workload_state(name, *SPECS[name])


def test_tiny_f32():
    st = _state("tiny_f32_n400_d16")
    check_end_to_end(st)
    check_oracle_codes(st)


def test_bf16_n1m():
    st = _state("bf16_n1m_d128_b16")
    check_end_to_end(st)
    check_oracle_codes(st)


@pytest.mark.timeout(900)
def test_bf16_n10m_headline_end_to_end():
    check_end_to_end(_state("bf16_n10m_d128_b256_excl5"))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("part", range(4))
def test_bf16_n10m_headline_oracle_codes(part):
    check_oracle_codes(_state("bf16_n10m_d128_b256_excl5"), part, 4)


@pytest.mark.timeout(900)
def test_fp8_n10m():
    st = _state("fp8_n10m_d256_b4096")
    check_end_to_end(st)
    check_oracle_codes(st)


@pytest.mark.timeout(1200)
def test_int8_n10m_end_to_end():
    check_end_to_end(_state("int8_n10m_d128_b256_excl5"))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("part", range(4))
def test_int8_n10m_oracle_codes(part):
    check_oracle_codes(_state("int8_n10m_d128_b256_excl5"), part, 4)


@pytest.mark.timeout(1500)
def test_bf16_n100m_end_to_end():
    check_end_to_end(_state("bf16_n100m_d64_b1024"))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("part", range(4))
def test_bf16_n100m_oracle_codes(part):
    check_oracle_codes(_state("bf16_n100m_d64_b1024"), part, 4)


@pytest.mark.timeout(1200)
def test_bf16_n10m_four_masks():
    """The headline corpus and batch with four result sets from one multi-mask pass: three
    disjoint item types (about 60%, 39% and 1% of the rows) and a random half, each with the
    workload's exclusion folded in. Every set equals mips_topk with that mask bitwise, and
    sampled queries equal the oracle's top-k under the mask."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from workloads import typed_masks
    dev = torch.device("cuda:0")
    w = WORKLOADS["bf16_n10m_d128_b256_excl5"]
    print("four masks: building inputs", flush=True)
    corpus, q, bm, codes, scale, q_or = build_both(w, dev)
    rows = typed_masks(w.n, bm)
    masks = torch.from_numpy(rows.view(np.int32)).to(dev)
    print("four masks: mips_topk_masks", flush=True)
    s, i = mips.topk_masks(q, corpus, masks, w.k)
    torch.cuda.synchronize()
    s, i = s.cpu().numpy(), i.cpu().numpy()
    sel = np.array([0, 77, 255], np.int64)
    ids_all = np.arange(w.n)
    for t in range(rows.shape[0]):
        s1, i1 = mips.topk(q, corpus, w.k, masks[t])
        torch.cuda.synchronize()
        assert np.array_equal(i1.cpu().numpy(), i[t])
        assert np.array_equal(s1.cpu().numpy().view(np.uint32), s[t].view(np.uint32))
        bad = ((rows[t][np.maximum(i[t], 0) >> 5] >> (np.maximum(i[t], 0) & 31).astype(np.uint32)) & 1) == 1
        assert not (bad & (i[t] >= 0)).any(), f"mask {t}: an excluded id was returned"
        print(f"four masks: oracle, mask {t}", flush=True)
        o_s, o_i = ref_topk(q_or[sel], w.query_dtype, codes, w.corpus_dtype, w.k,
                               exclude=rows[t], threads=threads())
        excluded = set(ids_all[((rows[t][ids_all >> 5] >> (ids_all & 31).astype(np.uint32)) & 1) == 1].tolist())
        stats = check_topk(s[t][sel], i[t][sel], o_s, o_i, q_or[sel], w.query_dtype, codes,
                           w.corpus_dtype, scale, excluded, w.n, TOL[w.corpus_dtype],
                           floor=floor_for(w.corpus_dtype, w.query_dtype))
        print(f"four masks: mask {t}: {stats}", flush=True)


def _bf16_close(got, want):
    """bf16 codes that differ by at most one step (fp32 normalisation on the GPU, fp64 in the
    oracle, each rounded to nearest even)."""
    gv, ov = oracle.decode(got, "bf16"), oracle.decode(want, "bf16")
    return np.all(np.abs(gv - ov) <= np.abs(ov) * 2.0 ** -7 + 1e-30)


@pytest.mark.timeout(600)
def test_row_kernels_past_the_launch_work_item_limit():
    """A launch counts its work-items in 32 bits, so row-wise kernels of more than 2^22
    workgroups go out as several launches: l2_normalize at 2^24 + 5 rows (4 rows per
    workgroup) and the index build at 2^27 + 40 rows (one 32-row block per workgroup, D=16
    bf16: 8.6 GB in, 4.3 GB out). Rows on both sides of each split, the first rows and the
    last (partial) block match the oracle. The input is a deterministic integer pattern
    built on the GPU; the oracle rebuilds the sampled rows on the host."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from tests.mips_check import untile
    from workloads import lattice_rows
    dev = torch.device("cuda:0")
    d = 16

    rows = 4 * (1 << 22) + 5
    print(f"launch split: l2_normalize rows={rows} d={d}", flush=True)
    x = lattice_rows(0, rows, d, dev)
    y = mips.l2_normalize(x, "f32")
    torch.cuda.synchronize()
    del x
    cut = 4 * (1 << 22)
    for r0, r1 in ((0, 3), (cut - 3, cut + 3), (rows - 2, rows)):
        want = oracle.normalize(lattice_rows(r0, r1, d))
        got = y[r0:r1].cpu().numpy().astype(np.float64)
        assert np.allclose(got, want, rtol=4e-7, atol=1e-30), (r0, r1)
    del y

    rows = 32 * (1 << 22) + 40
    nblk = (rows + 31) // 32
    print(f"launch split: prepare_corpus bf16 rows={rows} d={d} blocks={nblk}", flush=True)
    x = torch.empty(rows, d, dtype=torch.float32, device=dev)
    step = 1 << 24
    for r0 in range(0, rows, step):
        x[r0:r0 + step] = lattice_rows(r0, min(rows, r0 + step), d, dev)
    corpus = mips.prepare_corpus(x, "bf16")
    torch.cuda.synchronize()
    del x
    bb = 32 * d * 2
    for g in (0, (1 << 22) - 1, 1 << 22, nblk - 1):
        live = min(32, rows - 32 * g)
        got = untile(corpus.packed[g * bb:(g + 1) * bb].cpu().numpy(), 32, d, "bf16")
        want, _ = oracle.prepare(lattice_rows(32 * g, 32 * g + live, d), "bf16")
        assert _bf16_close(got[:live], want), f"block {g}"
        assert np.all(got[live:] == 0), f"block {g}: padding rows"
    del corpus
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_bf16_n_at_the_id_limit():
    """N = 2^31 - 65, the largest index the C ABI takes (int32 ids), at D=16 bf16 (68.7 GB
    packed). The rows follow workloads.lattice_rows, which repeats every P = 128 * 4093 rows,
    so every row but the planted ones scores exactly as its residue id mod P. Three query
    vectors are planted, one each in the last (ragged) block, in the block before it and at
    id 5. The exact top-K therefore merges the planted rows with the first duplicates of the
    best residues, whose exact scores the oracle computes on one period (523,904 rows).
    The check: the GPU's ids equal that list except swaps within tolerance of the K-th
    score, and every returned score is within tolerance of its row's exact score."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from workloads import Workload, lattice_rows
    dev = torch.device("cuda:0")
    n, d, k, P = (1 << 31) - 65, 16, 10, 128 * 4093
    assert n == 0x7FFFFFFF - 64
    qraw = Workload("planted", "clustered", n=64, d=d, b=3, k=k, corpus_dtype="bf16",
                    query_dtype="bf16", clusters=2, seed=31).queries()
    planted = [n - 1, n - 40, 5]  # planted[u] holds query u's raw vector
    print(f"id limit: building n={n} d={d} bf16 on the GPU", flush=True)
    corpus = mips.empty_corpus(n, d, "bf16", dev)
    step = 1 << 25
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        x = lattice_rows(r0, r1, d, dev)
        for u, p in enumerate(planted):
            if r0 <= p < r1:
                x[p - r0] = torch.from_numpy(qraw[u]).to(dev)
        mips.prepare_rows(corpus, x, r0)
        del x
    q = mips.l2_normalize(torch.from_numpy(qraw).to(dev), "bf16")
    print("id limit: mips_topk", flush=True)
    s, i = mips.topk(q, corpus, k)
    torch.cuda.synchronize()
    s, i = s.cpu().numpy(), i.cpu().numpy()
    del corpus
    torch.cuda.empty_cache()

    print("id limit: oracle on one period", flush=True)
    q_or, _ = oracle.prepare(qraw, "bf16")
    c_period, _ = oracle.prepare(lattice_rows(0, P, d), "bf16")
    c_planted, _ = oracle.prepare(qraw, "bf16")
    nres = 2 * k
    r_s, r_i = oracle.topk(q_or, "bf16", c_period, "bf16", nres, threads=threads())
    for t in range(3):
        ps = oracle.scores(q_or, "bf16", c_planted, "bf16", np.full(3, t), np.arange(3))
        cand = [(float(ps[u]), planted[u]) for u in range(3)]
        for sc, r in zip(r_s[t], r_i[t]):
            ids = [int(r) + m * P for m in range(k + 3)]
            cand += [(float(sc), j) for j in ids if j < n and j not in planted]
        cand.sort(key=lambda e: (-e[0], e[1]))
        want_s = np.array([e[0] for e in cand[:k]])
        want_i = np.array([e[1] for e in cand[:k]])
        # complete: residues past the first nres all score below the K-th entry
        assert r_s[t, -1] < want_s[-1], "too many residues tie at the K-th score"
        assert i[t, 0] == planted[t], (t, i[t])
        # every returned row's exact score, from its own codes
        for rank, (gs, gi) in enumerate(zip(s[t], i[t])):
            assert 0 <= gi < n
            if gi in planted:
                ex = float(ps[planted.index(gi)])
            else:
                ex = float(oracle.scores(q_or, "bf16", c_period, "bf16", np.array([t]),
                                         np.array([gi % P]))[0])
            assert abs(gs - ex) <= TOL["bf16"], (t, rank, gi, gs, ex)
        order_ok = (s[t][:-1] > s[t][1:]) | ((s[t][:-1] == s[t][1:]) & (i[t][:-1] < i[t][1:]))
        assert np.all(order_ok)
        diff = set(i[t].tolist()) ^ set(want_i.tolist())
        for gi in diff:
            ex = (float(ps[planted.index(gi)]) if gi in planted else
                  float(oracle.scores(q_or, "bf16", c_period, "bf16", np.array([t]),
                                      np.array([gi % P]))[0]))
            assert abs(ex - want_s[-1]) <= TOL["bf16"], f"query {t}: id {gi} swapped beyond tolerance"
        print(f"id limit: query {t}: ids {i[t][:4].tolist()}..., {len(diff) // 2} swaps", flush=True)
