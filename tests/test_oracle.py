"""Pins of the CPU oracle against facts that do not come from the oracle itself:
format definitions and library conversions, closed forms, invariants, and an exact
rational brute force on tiny inputs. CPU only."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, bitmap_from_ids


# ------------------------------------------------------------------ formats
def test_e4m3_decode_closed_forms():
    # OCP E4M3: bias 7, 3 mantissa bits, subnormal step 2^-9, max 448, 0x7F/0xFF NaN.
    assert oracle.e4m3_value(0x00) == 0.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x39) == 1.125
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0xFE) == -448.0
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))
    for c in range(0x7F):
        assert oracle.e4m3_value(c | 0x80) == -oracle.e4m3_value(c)


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan], mine[~nan])


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(-448, 448, 4000),
        rng.standard_normal(4000) * 2.0 ** rng.integers(-12, 6, 4000),
        # exact midpoints between neighbouring codes (ties go to even)
        [(oracle.e4m3_value(c) + oracle.e4m3_value(c + 1)) / 2 for c in range(0x7D)],
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3_from(x) for x in v.astype(np.float64)], np.uint8)
    assert np.array_equal(ref, mine)


def test_e4m3_encode_ties_and_saturation():
    assert oracle.e4m3_from(1.0 + 2 ** -4) == 0x38        # tie between 1 and 1.125 -> even (1)
    assert oracle.e4m3_from(1.0 + 3 * 2 ** -4) == 0x3A    # tie between 1.125 and 1.25 -> 1.25
    assert oracle.e4m3_from(460.0) == 0x7E                # saturates at 448
    assert oracle.e4m3_from(1e6) == 0x7E
    assert oracle.e4m3_from(-1e6) == 0xFE
    assert oracle.e4m3_from(2.0 ** -10) == 0x00           # tie between 0 and 2^-9 -> 0
    assert oracle.e4m3_from(3 * 2.0 ** -10) == 0x02       # tie between 2^-9 and 2^-8 -> 2^-8


def test_bf16_decode_and_encode_match_torch():
    codes = torch.arange(0, 65536, 7, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    mine = np.array([oracle.bf16_value(int(c) & 0xFFFF) for c in codes.numpy()])
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin], mine[fin])
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(5000) * 2.0 ** rng.integers(-130, 40, 5000),
                        rng.uniform(-1, 1, 5000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    mine = np.array([oracle.bf16_from(x) for x in v.astype(np.float64)], np.uint16)
    assert np.array_equal(ref, mine)


def test_bf16_encode_ties():
    assert oracle.bf16_from(1.0 + 2 ** -8) == 0x3F80        # tie -> even (1.0)
    assert oracle.bf16_from(1.0 + 3 * 2 ** -8) == 0x3F82    # tie -> even (1 + 2^-6)
    assert oracle.bf16_from(-0.0) == 0x8000


def test_e4m3_row_scale_rule():
    assert oracle.e4m3_row_scale(448.0) == 1.0
    assert oracle.e4m3_row_scale(449.0) == 2.0
    assert oracle.e4m3_row_scale(0.5) == 2.0 ** -9
    assert oracle.e4m3_row_scale(0.0) == 1.0
    rng = np.random.default_rng(3)
    for a in rng.uniform(1e-3, 1.0, 300):
        s = oracle.e4m3_row_scale(a)
        assert a <= 448 * s and a > 448 * s / 2
        assert np.log2(s) == np.round(np.log2(s))


def test_i8_encode_matches_torch_round_and_clip():
    # nearest integer with ties to even (torch.round), clipped to the symmetric range
    rng = np.random.default_rng(21)
    v = np.concatenate([rng.uniform(-140, 140, 5000), np.arange(-130, 131) + 0.5,
                        np.arange(-130, 131).astype(np.float64)])
    ref = torch.clamp(torch.round(torch.from_numpy(v)), -127, 127).to(torch.int8).numpy()
    mine = np.array([oracle.i8_from(x) for x in v], np.int8)
    assert np.array_equal(ref, mine)
    assert oracle.i8_from(2.5) == 2 and oracle.i8_from(3.5) == 4 and oracle.i8_from(-2.5) == -2
    assert oracle.i8_from(127.5) == 127 and oracle.i8_from(-1e9) == -127


def test_i8_row_scale_rule():
    assert oracle.i8_row_scale(127.0) == 1.0
    assert oracle.i8_row_scale(0.0) == float(np.float32(1e-12))
    rng = np.random.default_rng(22)
    for a in rng.uniform(1e-3, 1.0, 300):
        s = oracle.i8_row_scale(a)
        assert s == float(np.float32(a / 127))
        # the largest element maps to +-127 (up to the float rounding of the scale)
        assert oracle.i8_from(a / s) == 127


# ------------------------------------------------------------- normalisation
def test_normalize_closed_forms():
    y = oracle.normalize(np.array([[3, 4], [0, 0], [1e-7, 1e-7]], np.float32))
    assert np.allclose(y[0], [0.6, 0.8], rtol=0, atol=1e-16)
    assert np.array_equal(y[1], [0.0, 0.0])
    # sum of squares 2e-14 < 1e-12: the norm is clamped to sqrt(1e-12) = 1e-6
    x2 = np.float64(np.float32(1e-7))
    assert np.allclose(y[2], [x2 / 1e-6, x2 / 1e-6], rtol=1e-15)


def test_normalize_matches_numpy_norm():
    x = np.random.default_rng(4).standard_normal((200, 37)).astype(np.float32)
    y = oracle.normalize(x)
    ref = x.astype(np.float64) / np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True)
    assert np.allclose(y, ref, rtol=1e-14, atol=0)


@pytest.mark.parametrize("dtype,tol", [("f32", 1e-6), ("bf16", 2 ** -7), ("fp8", 2 ** -3),
                                       ("int8", 2 ** -5)])
def test_prepare_unit_norm_and_elementwise(dtype, tol):
    x = np.random.default_rng(5).standard_normal((300, 64)).astype(np.float32)
    codes, scale = oracle.prepare(x, dtype)
    v = oracle.decode(codes, dtype, scale)
    y = oracle.normalize(x)
    # The row is normalised in binary32 (unit roundoff u = 2^-24): a d-term running sum of
    # rounded squares, a square root and a quotient put y32 within (d/2 + 3) u of the exact y.
    # Every stored element is then within half a step of y32.
    g = (x.shape[1] / 2 + 3) * 2.0 ** -24
    if dtype == "f32":
        assert np.all(np.abs(v - y) <= g * np.abs(y))
    elif dtype == "bf16":
        assert np.all(np.abs(v - y) <= np.abs(y) * (2 ** -8 + 2 * g) + 2.0 ** -134)
    elif dtype == "int8":
        # half a code step of the row's scale (the quotient y32 / s adds at most 127 u of a
        # step); the largest element of every row is +-127
        sc = scale[:, None].astype(np.float64)
        assert np.all(np.abs(v - y) <= sc * (0.5 + 128 * 2.0 ** -24) + g * np.abs(y))
        assert np.all(np.abs(codes.astype(np.int32)).max(axis=1) == 127)
        assert np.all(np.abs(codes.astype(np.int32)) <= 127)
    else:
        step = np.maximum(np.abs(y / scale[:, None]), 2.0 ** -6)
        ulp = 2.0 ** (np.floor(np.log2(step)) - 3)
        assert np.all(np.abs(v / scale[:, None] - y / scale[:, None])
                      <= ulp / 2 + g * np.abs(y / scale[:, None]) + 1e-18)
        assert np.all(np.abs(v / scale[:, None]).max(axis=1) <= 448)
    norms = np.linalg.norm(v, axis=1)
    assert np.all(np.abs(norms - 1) <= tol)


# ------------------------------------------------------------------ top-k
def _fraction_topk(qv, cv, k, excluded=()):
    """Exact rational brute force: Fractions, Python's sorted with a (-score, id) key."""
    qf = [[Fraction(float(a)) for a in row] for row in qv]
    cf = [[Fraction(float(a)) for a in row] for row in cv]
    out = []
    for q in qf:
        sc = [(sum(a * b for a, b in zip(q, c)), i) for i, c in enumerate(cf) if i not in excluded]
        sc = sorted(sc, key=lambda t: (-t[0], t[1]))[:k]
        out.append(sc)
    return out


@pytest.mark.parametrize("c_dtype,q_dtype", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16"),
                                             ("bf16", "f32"), ("int8", "bf16"), ("int8", "f32")])
@pytest.mark.parametrize("with_exclusion", [False, True])
def test_topk_matches_exact_rational_bruteforce(c_dtype, q_dtype, with_exclusion):
    rng = np.random.default_rng(6)
    n, d, b, k = 90, 12, 5, 17
    x = rng.standard_normal((n, d)).astype(np.float32)
    corpus, scale = oracle.prepare(x, c_dtype)
    qraw = rng.standard_normal((b, d)).astype(np.float32)
    queries, _ = oracle.prepare(qraw, q_dtype)
    excl = set(rng.choice(n, 20, replace=False).tolist()) if with_exclusion else set()
    bitmap = bitmap_from_ids(np.array(sorted(excl), np.int64), n) if excl else None
    s, ids = oracle.topk(queries, q_dtype, corpus, c_dtype, k, row_scale=scale, exclude=bitmap,
                         threads=3)
    ref = _fraction_topk(oracle.decode(queries, q_dtype), oracle.decode(corpus, c_dtype, scale),
                         k, excl)
    for qi in range(b):
        assert ids[qi].tolist() == [i for _, i in ref[qi]]
        assert np.allclose(s[qi], [float(v) for v, _ in ref[qi]], rtol=1e-15, atol=1e-17)


def test_topk_identity_corpus():
    d = 16
    corpus = np.eye(d, dtype=np.float32)
    for j in range(d):
        q = np.zeros((1, d), np.float32)
        q[0, j] = 1.0
        s, ids = oracle.topk(q, "f32", corpus, "f32", d)
        assert ids[0, 0] == j and s[0, 0] == 1.0
        assert ids[0, 1:].tolist() == [i for i in range(d) if i != j]
        assert np.all(s[0, 1:] == 0.0)


def test_topk_all_equal_corpus_tie_rule_and_exclusion():
    n, d, k = 300, 8, 25
    corpus = np.full((n, d), 0x3E80, np.uint16)  # every element 0.25
    q = np.full((2, d), 0x3E80, np.uint16)
    s, ids = oracle.topk(q, "bf16", corpus, "bf16", k)
    assert np.all(ids == np.arange(k)) and np.all(s == d * 0.0625)
    excl = np.array([0, 3, 4, 31, 32, 33, 64], np.int64)
    s, ids = oracle.topk(q, "bf16", corpus, "bf16", k, exclude=bitmap_from_ids(excl, n))
    expect = [i for i in range(n) if i not in set(excl.tolist())][:k]
    assert ids[0].tolist() == expect and ids[1].tolist() == expect


def test_exclusion_bit_order():
    n = 100
    bm = bitmap_from_ids(np.array([33]), n)
    assert bm[1] == 2 and bm.sum() == 2
    corpus = np.zeros((n, 4), np.float32)
    corpus[33] = 1.0
    corpus[34] = 0.5
    s, ids = oracle.topk(np.ones((1, 4), np.float32), "f32", corpus, "f32", 1, exclude=bm)
    assert ids[0, 0] == 34


def _grid_inputs(rng, n, d, b):
    """bf16-representable values on a coarse grid: every dot product is exact in any order."""
    cv = rng.integers(-4, 5, (n, d)).astype(np.float32) / 4
    qv = rng.integers(-4, 5, (b, d)).astype(np.float32) / 4
    to16 = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return to16(cv), to16(qv), cv.astype(np.float64), qv.astype(np.float64)


def test_full_order_matches_numpy_lexsort_and_negation():
    rng = np.random.default_rng(7)
    n, d, b = 400, 8, 4
    c16, q16, cv, qv = _grid_inputs(rng, n, d, b)
    sc = qv @ cv.T
    s, ids = oracle.topk(q16, "bf16", c16, "bf16", n)
    for qi in range(b):
        order = np.lexsort((np.arange(n), -sc[qi]))
        assert np.array_equal(ids[qi], order)
        assert np.array_equal(s[qi], sc[qi][order])
    # negated query: its full order is the bottom-up order of the original scores
    neg = (q16 ^ np.uint16(0x8000))
    s2, ids2 = oracle.topk(neg, "bf16", c16, "bf16", n)
    for qi in range(b):
        assert np.array_equal(ids2[qi], np.lexsort((np.arange(n), sc[qi])))
        assert np.array_equal(s2[qi], -sc[qi][ids2[qi]])


def test_k_larger_than_eligible_pads():
    corpus = np.eye(4, dtype=np.float32)
    s, ids = oracle.topk(np.ones((1, 4), np.float32), "f32", corpus, "f32", 7,
                         exclude=bitmap_from_ids(np.array([2]), 4))
    assert ids[0].tolist() == [0, 1, 3, -1, -1, -1, -1]
    assert np.all(np.isneginf(s[0, 3:]))


def _small_clustered(n=3000, d=32, b=6, clusters=40, seed=11):
    w = WORKLOADS["bf16_n1m_d128_b16"].replace(n=n, d=d, b=b, clusters=clusters, seed=seed)
    corpus, _ = oracle.prepare(w.corpus(), "bf16")
    queries, _ = oracle.prepare(w.queries(), "bf16")
    return w, corpus, queries


def test_k_prefix_and_exclusion_shift():
    w, corpus, queries = _small_clustered()
    s1, i1 = oracle.topk(queries, "bf16", corpus, "bf16", 30)
    s2, i2 = oracle.topk(queries, "bf16", corpus, "bf16", 31)
    assert np.array_equal(i1, i2[:, :30]) and np.array_equal(s1, s2[:, :30])
    for qi in range(queries.shape[0]):
        bm = bitmap_from_ids(np.array([i2[qi, 0]]), w.n)
        s3, i3 = oracle.topk(queries[qi:qi + 1], "bf16", corpus, "bf16", 30, exclude=bm)
        assert np.array_equal(i3[0], i2[qi, 1:31]) and np.array_equal(s3[0], s2[qi, 1:31])


def test_permutation_invariance():
    w, corpus, queries = _small_clustered(seed=12)
    perm = np.random.default_rng(13).permutation(w.n)
    s1, i1 = oracle.topk(queries, "bf16", corpus, "bf16", 50)
    s2, i2 = oracle.topk(queries, "bf16", corpus[perm], "bf16", 50)
    assert np.array_equal(s1, s2)           # score lists bitwise identical
    for qi in range(queries.shape[0]):
        untied = np.concatenate([[True], s1[qi, 1:] != s1[qi, :-1]]) & \
            np.concatenate([s1[qi, :-1] != s1[qi, 1:], [True]])
        assert np.array_equal(perm[i2[qi]][untied], i1[qi][untied])
        assert set(perm[i2[qi]].tolist()) == set(i1[qi].tolist()) or s1[qi, -1] == s1[qi, -2]


def test_planted_item_and_score_bound():
    w, _, _ = _small_clustered(seed=14)
    x = w.corpus()
    qraw = w.queries()
    for qi, p in enumerate([5, 777, 2999]):
        xp = x.copy()
        xp[p] = qraw[qi]
        corpus, _ = oracle.prepare(xp, "bf16")
        q, _ = oracle.prepare(qraw[qi:qi + 1], "bf16")
        s, ids = oracle.topk(q, "bf16", corpus, "bf16", 5)
        assert ids[0, 0] == p
        assert s[0, 0] > s[0, 1] + 0.02
        qv = oracle.decode(q, "bf16")[0]
        assert abs(s[0, 0] - float(qv @ qv)) < 1e-12
        # normalised bf16 rows: every score within (1 + 2^-8)^2 of the unit bound
        assert np.all(np.abs(s) <= (1 + 2 ** -8) ** 2)


def test_tiny_workload_groups():
    """The toy corpus: each query's best items belong to its own taste group."""
    w = WORKLOADS["tiny_f32_n400_d16"]
    corpus, _ = oracle.prepare(w.corpus(), "f32")
    queries, _ = oracle.prepare(w.queries(), "f32")
    s, ids = oracle.topk(queries, "f32", corpus, "f32", w.k)
    g = w.query_clusters()
    assert np.mean(ids % 8 == g[:, None]) > 0.95
    assert np.all(s[:, :-1] >= s[:, 1:])


# ------------------------------------------------------------------ merging
@pytest.mark.parametrize("cuts", [(0, 130, 131, 400), (0, 7, 400), (0, 200, 260, 300, 399, 400)])
def test_merge_of_shard_topk_equals_full_topk(cuts):
    """Top-k decomposes over a row partition: merging the shards' own top-k lists (ids
    shifted by each shard's first row) gives the whole corpus's top-k, ties included."""
    rng = np.random.default_rng(23)
    n, d, b, k = 400, 8, 5, 40
    c16, q16, _, _ = _grid_inputs(rng, n, d, b)   # many exact ties across shards
    full_s, full_i = oracle.topk(q16, "bf16", c16, "bf16", k)
    lists_s, lists_i = [], []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        s, i = oracle.topk(q16, "bf16", c16[lo:hi], "bf16", k)
        lists_s.append(s.astype(np.float32))
        lists_i.append(i)
    ms, mi = oracle.merge_topk(np.stack(lists_s), np.stack(lists_i), np.array(cuts[:-1]), k)
    assert np.array_equal(mi, full_i)
    assert np.array_equal(ms, full_s.astype(np.float32))


def test_merge_pads_and_skips_padding():
    s = np.array([[[0.5, -np.inf, -np.inf]], [[0.7, 0.5, -np.inf]]], np.float32)
    i = np.array([[[3, -1, -1]], [[0, 1, -1]]], np.int32)
    ms, mi = oracle.merge_topk(s, i, np.array([0, 100]), 5)
    assert mi[0].tolist() == [100, 3, 101, -1, -1]      # 0.7, then the 0.5 tie by id
    assert ms[0, :3].tolist() == [np.float32(0.7), 0.5, 0.5]
    assert np.all(np.isneginf(ms[0, 3:]))


# ------------------------------------------------------------ multi-interest
def test_maxsim_reduces_to_topk():
    """One interest vector is the plain top-k; a user whose vectors repeat one query is
    that query's top-k (the max of equal scores)."""
    w, corpus, queries = _small_clustered(seed=24)
    s1, i1 = oracle.topk(queries, "bf16", corpus, "bf16", 25)
    s2, i2 = oracle.maxsim_topk(queries[:, None, :], "bf16", corpus, "bf16", 25)
    assert np.array_equal(i1, i2) and np.array_equal(s1, s2)
    rep = np.repeat(queries[:, None, :], 3, axis=1)
    s3, i3 = oracle.maxsim_topk(rep, "bf16", corpus, "bf16", 25)
    assert np.array_equal(i1, i3) and np.array_equal(s1, s3)


def test_maxsim_closed_form_two_interests():
    """Interests e_0 and e_1 over axis-aligned items: the items of both axes come first,
    ordered by their own coordinate, ties by id."""
    d = 4
    corpus = np.zeros((8, d), np.float32)
    vals = [0.9, 0.5, 0.7, 0.3]
    for j, v in enumerate(vals):
        corpus[j, 0] = v           # ids 0..3 on axis 0
        corpus[4 + j, 1] = v       # ids 4..7 on axis 1
    corpus[:, 2] = 0.1             # every item also has a small third coordinate
    q = np.zeros((1, 2, d), np.float32)
    q[0, 0, 0] = 1.0
    q[0, 1, 1] = 1.0
    s, ids = oracle.maxsim_topk(q, "f32", corpus, "f32", 8)
    assert ids[0].tolist() == [0, 4, 2, 6, 1, 5, 3, 7]
    assert np.allclose(s[0], [0.9, 0.9, 0.7, 0.7, 0.5, 0.5, 0.3, 0.3])


def test_maxsim_equals_brute_force_max():
    rng = np.random.default_rng(25)
    n, d, b, m, k = 200, 12, 3, 4, 30
    corpus, _ = oracle.prepare(rng.standard_normal((n, d)).astype(np.float32), "bf16")
    q, _ = oracle.prepare(rng.standard_normal((b * m, d)).astype(np.float32), "bf16")
    s, ids = oracle.maxsim_topk(q.reshape(b, m, d), "bf16", corpus, "bf16", k)
    cv, qv = oracle.decode(corpus, "bf16"), oracle.decode(q, "bf16").reshape(b, m, d)
    for u in range(b):
        best = (qv[u] @ cv.T).max(axis=0)
        order = sorted(range(n), key=lambda i: (-best[i], i))[:k]
        assert ids[u].tolist() == order


# ------------------------------------------------ quantised scoring (int8 branch)
def _rn32(fr: Fraction) -> np.float32:
    """Nearest binary32 to an exact rational, ties to even, found by comparing exact
    distances to the neighbours of a first guess (independent of any float multiply)."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))


def _torch_quantize_i8(u32: np.ndarray):
    """The per-user rule with torch's float32 ops: scale max(max|u|/127, 1e-12), codes
    round-half-even(u / scale) clipped to [-127, 127]."""
    t = torch.from_numpy(np.ascontiguousarray(u32, np.float32))
    us = torch.clamp(t.abs().amax(dim=1) / 127.0, min=1e-12)
    uq = torch.clamp(torch.round(t / us[:, None]), -127, 127).to(torch.int32)
    return uq.numpy(), us.numpy()


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_quantize_int8_matches_torch(x_dtype):
    rng = np.random.default_rng(40)
    u = rng.standard_normal((400, 64)).astype(np.float32) * rng.uniform(1e-3, 2, (400, 1)).astype(np.float32)
    # exact half steps: with max 127 * 2^-7 the scale is 2^-7 and (j + 0.5) 2^-7 is a tie
    u[0] = 0.0
    u[0, 0] = 127 * 2.0 ** -7
    u[0, 1:12] = (np.arange(-6, 5) + 0.5) * 2.0 ** -7
    u[1] = 0.0                                     # zero row: scale 1e-12, codes 0
    u[2] = 0.0
    u[2, 3] = -0.5 * np.float32(1e-12)             # below the floor: -0.5 steps -> 0 (even)
    x = u if x_dtype == "f32" else torch.from_numpy(u).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vals = oracle.decode(x, x_dtype).astype(np.float32)
    codes, scale = oracle.quantize(x, x_dtype, "int8")
    ref_q, ref_s = _torch_quantize_i8(vals)
    assert np.array_equal(scale.view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(codes.astype(np.int32), ref_q)
    assert scale[0] == 2.0 ** -7 and codes[0, 0] == 127
    assert codes[0, 1:12].tolist() == [-6, -4, -4, -2, -2, 0, 0, 2, 2, 4, 4]
    assert scale[1] == np.float32(1e-12) and not codes[1].any()
    if x_dtype == "f32":
        assert scale[2] == np.float32(1e-12) and not codes[2].any()


def test_quantize_fp8_matches_torch_float8():
    rng = np.random.default_rng(41)
    u = (rng.standard_normal((300, 128)) * rng.uniform(1e-3, 3, (300, 1))).astype(np.float32)
    u[7] = 0.0
    codes, scale = oracle.quantize(u, "f32", "fp8")
    for r in range(u.shape[0]):
        s = scale[r]
        assert s == oracle.e4m3_row_scale(float(np.abs(u[r]).max()))   # the pinned scale rule
        ref = torch.from_numpy(u[r] / s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes[r], ref), r
    assert scale[7] == 1.0 and not codes[7].any()


def _int8_bruteforce(qvals, cq, cs, k, excluded=()):
    """The quantised branch from pinned pieces: torch's quantisation of the queries, Python
    integer dot products, and each product rounded to binary32 by exact rationals (user
    scale first, then the item scale); sorted by (-score, id)."""
    uq, us = _torch_quantize_i8(qvals)
    out = []
    for qi in range(uq.shape[0]):
        row = []
        for i in range(cq.shape[0]):
            if i in excluded:
                continue
            acc = sum(int(a) * int(c) for a, c in zip(uq[qi], cq[i]))
            t = _rn32(Fraction(acc) * Fraction(float(us[qi])))
            row.append((float(_rn32(Fraction(float(t)) * Fraction(float(cs[i])))), i))
        out.append(sorted(row, key=lambda e: (-e[0], e[1]))[:k])
    return out


@pytest.mark.parametrize("q_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("with_exclusion", [False, True])
def test_topk_int8_matches_integer_bruteforce(q_dtype, with_exclusion):
    rng = np.random.default_rng(42)
    n, d, b, k = 70, 16, 4, 15
    cq, cs = oracle.prepare(rng.standard_normal((n, d)).astype(np.float32), "int8")
    q, _ = oracle.prepare(rng.standard_normal((b, d)).astype(np.float32), q_dtype)
    # two rows with identical codes and scales tie exactly: the lower id comes first
    cq[40], cs[40] = cq[3], cs[3]
    excl = set(rng.choice(n, 12, replace=False).tolist()) - {3, 40} if with_exclusion else set()
    bitmap = bitmap_from_ids(np.array(sorted(excl), np.int64), n) if excl else None
    s, ids = oracle.topk_int8(q, q_dtype, cq, k, cs, exclude=bitmap, threads=2)
    ref = _int8_bruteforce(oracle.decode(q, q_dtype).astype(np.float32), cq, cs, k, excl)
    for qi in range(b):
        assert ids[qi].tolist() == [i for _, i in ref[qi]]
        assert s[qi].tolist() == [v for v, _ in ref[qi]]
        pos = {i: p for p, i in enumerate(ids[qi].tolist())}
        if 3 in pos and 40 in pos:
            assert pos[3] < pos[40]
    # scores_int8 of the returned pairs is bitwise the listed score
    qidx = np.repeat(np.arange(b), k)
    e = oracle.scores_int8(q, q_dtype, cq, cs, qidx, ids.ravel())
    assert np.array_equal(e, s.ravel())


def test_int8_scores_round_the_exact_score_when_the_user_scale_is_a_power_of_two():
    """u = m 2^-e with max|m| = 127 makes the user scale exactly 2^-e and the codes exactly m,
    so the first product is exact and the score is the exact inner product of u with the
    stored row rounded once to binary32; that exact value is the unquantised oracle's."""
    rng = np.random.default_rng(43)
    n, d, b = 200, 32, 6
    cq, cs = oracle.prepare(rng.standard_normal((n, d)).astype(np.float32), "int8")
    m = rng.integers(-127, 128, (b, d))
    m[np.arange(b), rng.integers(0, d, b)] = np.where(rng.random(b) < 0.5, 127, -127)
    e = rng.integers(5, 12, b)
    u = (m * 2.0 ** -e[:, None]).astype(np.float32)
    s, ids = oracle.topk_int8(u, "f32", cq, n, cs, threads=2)
    exact = oracle.scores(u, "f32", cq, "int8", np.repeat(np.arange(b), n), ids.ravel(),
                          row_scale=cs).reshape(b, n)
    assert np.array_equal(s.astype(np.float32), exact.astype(np.float32))
    # the integer dot product itself, with power-of-two row scales as well
    cs2 = (2.0 ** -rng.integers(6, 9, n)).astype(np.float32)
    s2 = oracle.scores_int8(u, "f32", cq, cs2, np.repeat(np.arange(b), n), np.tile(np.arange(n), b))
    acc = (m.astype(np.int64) @ cq.astype(np.int64).T).ravel()
    assert np.array_equal(s2, acc * 2.0 ** -np.repeat(e, n) * np.tile(cs2.astype(np.float64), b))


def test_int8_scores_within_the_quantisation_bound_of_the_exact_score():
    """Rounding u_d to the nearest code moves it by at most half a step us/2, so the score
    differs from the exact inner product of the unquantised query with the stored row by at
    most (us/2) sum_d |c_d| s plus two binary32 roundings; a wrong scale or index would not."""
    rng = np.random.default_rng(44)
    n, d, b = 300, 128, 8
    cq, cs = oracle.prepare(rng.standard_normal((n, d)).astype(np.float32), "int8")
    q, _ = oracle.prepare(rng.standard_normal((b, d)).astype(np.float32), "bf16")
    s, ids = oracle.topk_int8(q, "bf16", cq, n, cs, threads=2)
    qv = oracle.decode(q, "bf16")
    exact = oracle.scores(q, "bf16", cq, "int8", np.repeat(np.arange(b), n), ids.ravel(),
                          row_scale=cs).reshape(b, n)
    us = np.maximum(np.abs(qv).max(axis=1) / 127, 1e-12)
    l1 = np.abs(cq.astype(np.float64))[ids].sum(axis=2) * cs[ids]
    bound = us[:, None] / 2 * l1 * (1 + 1e-6) + 2.0 ** -22 * np.abs(exact)
    assert np.all(np.abs(s - exact) <= bound)
    assert np.abs(s - exact).max() > 1e-5          # the quantisation is really applied


# ------------------------------------------------------- exact scores by pair
def test_scores_of_pairs_match_numpy_and_topk():
    rng = np.random.default_rng(45)
    n, d, b, k = 150, 24, 7, 40
    for c_dtype, q_dtype in (("bf16", "bf16"), ("fp8", "bf16"), ("f32", "f32"), ("int8", "f32")):
        cq, cs = oracle.prepare(rng.standard_normal((n, d)).astype(np.float32), c_dtype)
        q, _ = oracle.prepare(rng.standard_normal((b, d)).astype(np.float32), q_dtype)
        # arbitrary (query, id) pairs in a shuffled order: numpy's dot of the decoded rows
        qidx = rng.integers(0, b, 500)
        ids = rng.integers(0, n, 500)
        e = oracle.scores(q, q_dtype, cq, c_dtype, qidx, ids, row_scale=cs)
        ref = np.einsum("td,td->t", oracle.decode(q, q_dtype)[qidx],
                        oracle.decode(cq, c_dtype, cs)[ids])
        assert np.allclose(e, ref, rtol=1e-13, atol=1e-16), c_dtype
        # a wrong query or row index would show: the pairs really differ
        assert np.abs(ref - ref[rng.permutation(500)]).max() > 1e-2
        # and topk's scores are bitwise the scores of its own ids
        s, i = oracle.topk(q, q_dtype, cq, c_dtype, k, row_scale=cs, threads=2)
        e2 = oracle.scores(q, q_dtype, cq, c_dtype, np.repeat(np.arange(b), k), i.ravel(),
                           row_scale=cs)
        assert np.array_equal(e2, s.ravel()), c_dtype


# -------------------------------------------------- rows below the norm floor
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "int8"])
def test_prepare_rows_below_the_norm_floor(dtype):
    """Rows with sum x^2 < 1e-12 are divided by sqrt(1e-12) (the clamp); a zero row stays
    zero (fp8 scale 1, int8 scale 1e-12). Reference: torch's float32 ops, whose sums of
    these rows are exact, and torch's own bf16 / E4M3 / round conversions."""
    x = np.zeros((4, 32), np.float32)
    x[1, 0] = 1e-7
    x[2, 0], x[2, 5] = 3e-7, -4e-7
    x[3, :] = 1e-8
    codes, scale = oracle.prepare(x, dtype)
    t = torch.from_numpy(x)
    ss = torch.clamp((t * t).sum(dim=1, keepdim=True), min=1e-12)
    y = t / torch.sqrt(ss)
    assert float(ss[1, 0]) < 1e-12 or float(ss[1, 0]) == np.float32(1e-12)
    if dtype == "f32":
        assert np.array_equal(codes.view(np.uint32), y.numpy().view(np.uint32))
    elif dtype == "bf16":
        assert np.array_equal(codes, y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    elif dtype == "fp8":
        amax = y.abs().amax(dim=1).numpy()
        want_s = np.array([oracle.e4m3_row_scale(float(a)) for a in amax], np.float32)
        assert np.array_equal(scale, want_s) and scale[0] == 1.0
        ref = (y / torch.from_numpy(want_s)[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, ref)
    else:
        ref_q, ref_s = _torch_quantize_i8(y.numpy())
        assert np.array_equal(scale.view(np.uint32), ref_s.view(np.uint32))
        assert np.array_equal(codes.astype(np.int32), ref_q)
        assert scale[0] == np.float32(1e-12)
    assert not np.any(codes[0])


def test_maxsim_int8_reduces_to_topk_int8_and_takes_the_max():
    rng = np.random.default_rng(46)
    n, d, b, m, k = 120, 32, 3, 3, 25
    cq, cs = oracle.prepare(rng.standard_normal((n, d)).astype(np.float32), "int8")
    q, _ = oracle.prepare(rng.standard_normal((b * m, d)).astype(np.float32), "bf16")
    s1, i1 = oracle.maxsim_topk_int8(q.reshape(b * m, 1, d), "bf16", cq, k, cs)
    s2, i2 = oracle.topk_int8(q, "bf16", cq, k, cs)
    assert np.array_equal(i1, i2) and np.array_equal(s1, s2)
    s, i = oracle.maxsim_topk_int8(q.reshape(b, m, d), "bf16", cq, k, cs)
    for u in range(b):
        per = np.stack([oracle.scores_int8(q, "bf16", cq, cs, np.full(n, u * m + v), np.arange(n))
                        for v in range(m)])
        best = per.max(axis=0)
        order = sorted(range(n), key=lambda j: (-best[j], j))[:k]
        assert i[u].tolist() == order and s[u].tolist() == best[order].tolist()


def _absmax_e4m3(y: np.ndarray):
    """The other fp8 reading: scale max|y| / 448 per row, codes RNE-rounded E4M3 of y / scale
    (torch's float8_e4m3fn cast, clamped to the format's +-448 first). Decoded values."""
    amax = np.abs(y).max(axis=1, keepdims=True)
    s = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    v = np.clip(y / s, -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return codes * s.astype(np.float64)


def test_fp8_power_of_two_scale_error_budget():
    """The fp8 scale reading (a power of two per row, the smallest with max|y| <= 448 s)
    against a plain max|y| / 448 scale, on the fp8 workload's clustered generator (D=256):
    score errors of the quantised operands against the exact score of the normalised rows.
    E4M3 is a floating-point code, so a power-of-two scale only moves where a row's values fall
    on the exponent grid: its errors match the plain rule's (RMS 2.4e-3 against 2.3e-3, max
    1.2e-2 for both here), far inside the 6e-2 score tolerance."""
    w = WORKLOADS["fp8_n10m_d256_b4096"].replace(n=30000, b=48)
    x = w.corpus()
    qraw = w.queries()
    y = oracle.normalize(x.astype(np.float64))
    u = oracle.normalize(qraw.astype(np.float64))
    exact = u @ y.T
    # power-of-two rule, as stored by prepare (rows) and as the queries are quantised
    c_codes, c_scale = oracle.prepare(x, "fp8")
    q_codes, q_scale = oracle.quantize(u.astype(np.float32), "f32", "fp8")
    yp = oracle.decode(c_codes, "fp8", c_scale)
    up = oracle.decode(q_codes, "fp8", q_scale)
    assert np.all(np.log2(c_scale) == np.round(np.log2(c_scale)))
    # plain rule
    ya = _absmax_e4m3(y.astype(np.float32))
    ua = _absmax_e4m3(u.astype(np.float32))
    err = {"pow2": np.abs(up @ yp.T - exact), "absmax": np.abs(ua @ ya.T - exact),
           "pow2, f32 queries": np.abs(u @ yp.T - exact)}
    rms = {k: float(np.sqrt(np.mean(v * v))) for k, v in err.items()}
    mx = {k: float(v.max()) for k, v in err.items()}
    print({k: (f"rms {rms[k]:.2e}", f"max {mx[k]:.2e}") for k in err})
    assert mx["pow2"] < 2.0e-2 and mx["pow2, f32 queries"] < 2.0e-2   # tolerance: 6e-2
    assert rms["pow2"] <= 1.25 * rms["absmax"]
    assert mx["pow2"] <= 1.5 * mx["absmax"]
    # the element step: a power-of-two scale leaves the largest element in [224, 448] s
    lead = np.abs(y).max(axis=1) / c_scale
    assert lead.min() >= 224.0 * (1 - 2 ** -20) and lead.max() <= 448.0
