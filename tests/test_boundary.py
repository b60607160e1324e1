"""The C ABI without a GPU: the library loads, exports every entry point include/mips.h
declares, sizes its buffers as documented, and rejects invalid arguments before any HIP
call (nothing here launches a kernel)."""
import ctypes as C
import os
import re

import pytest

import exact_inner_product_amd as mips
from tests.mips_check import untile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mips.h")

F32, BF16, FP8, INT8 = 0, 1, 2, 3
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mips.LIB_PATH):
        from exact_inner_product_amd import build
        build.build()
    return mips.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mips_[a-z0-9_]+)\s*\(", text)))


def test_header_and_exports(L):
    names = declared_functions()
    assert set(names) == set(mips.EXPORTS)
    for name in names:
        assert hasattr(L, name), name
    assert mips.lib().mips_status_string(3).decode() == "workspace too small"


def test_corpus_bytes(L):
    assert L.mips_corpus_bytes(1, 128, BF16) == 32 * 128 * 2
    assert L.mips_corpus_bytes(33, 128, BF16) == 64 * 128 * 2
    assert L.mips_corpus_bytes(10_000_000, 128, BF16) == 10_000_000 * 256
    assert L.mips_corpus_bytes(100, 256, FP8) == 128 * 256
    assert L.mips_corpus_bytes(100, 16, FP8) == -1      # fp8 needs d in {64, 128, 256}
    assert L.mips_corpus_bytes(100, 48, BF16) == -1
    assert L.mips_corpus_bytes(0, 128, BF16) == -1
    assert L.mips_scale_count(1) == 32 and L.mips_scale_count(64) == 64
    assert L.mips_corpus_bytes(100, 32, INT8) == 128 * 32
    assert L.mips_corpus_bytes(100, 16, INT8) == -1     # int8 needs d in {32, .., 256}


def test_workspace_size(L):
    ws = L.mips_topk_workspace_size(256, 10_000_000, 128, 500, BF16, BF16)
    assert ws > 256 * 32768 * 8
    assert ws < 1 << 30
    assert L.mips_topk_workspace_size(0, 100, 128, 10, BF16, BF16) == 0
    assert L.mips_topk_workspace_size(4, 100, 128, 1025, BF16, BF16) == 0
    assert L.mips_topk_workspace_size(4, 100, 48, 10, BF16, BF16) == 0
    assert L.mips_topk_workspace_size(4, 100, 128, 10, BF16, F32) == 0  # bf16 queries need a bf16/fp8 corpus
    # an explicit capacity: more candidates, more bytes; 0 for a capacity below 1
    small = L.mips_topk_workspace_size_for(256, 10_000_000, 128, 500, BF16, BF16, 1)
    big = L.mips_topk_workspace_size_for(256, 10_000_000, 128, 500, BF16, BF16, 1 << 16)
    assert 0 < small < ws < big
    assert big - small >= 256 * ((1 << 16) - 1024) * 8
    assert L.mips_topk_workspace_size_for(256, 10_000_000, 128, 500, BF16, BF16, 0) == 0


def _topk(L, q=0x1000, qdt=BF16, b=4, corpus=0x2000, scale=None, cdt=BF16, n=1000, d=128,
          excl=None, rw=0, k=10, out_s=0x3000, out_i=0x4000, ws=0x10000, wsb=1 << 30):
    vp = lambda x: None if x is None else C.c_void_p(x)
    return L.mips_topk(vp(q), qdt, b, vp(corpus), vp(scale), cdt, n, d, vp(excl), rw, k,
                       vp(out_s), vp(out_i), vp(ws), wsb, None)


def test_topk_argument_validation(L):
    assert _topk(L, q=None) == INVALID
    assert _topk(L, corpus=None) == INVALID
    assert _topk(L, out_s=None) == INVALID
    assert _topk(L, ws=None) == INVALID
    assert _topk(L, b=0) == INVALID
    assert _topk(L, n=0) == INVALID
    assert _topk(L, k=0) == INVALID
    assert _topk(L, k=1025) == UNSUPPORTED
    assert _topk(L, d=48) == UNSUPPORTED
    assert _topk(L, cdt=FP8, d=32, scale=0x5000) == UNSUPPORTED
    assert _topk(L, cdt=FP8) == INVALID                 # fp8 needs row_scale
    assert _topk(L, qdt=7) == UNSUPPORTED
    assert _topk(L, cdt=F32) == UNSUPPORTED             # f32 corpus needs f32 queries
    assert _topk(L, corpus=0x2008) == INVALID           # corpus must be 16-byte aligned
    assert _topk(L, ws=0x10010) == INVALID              # workspace must be 256-byte aligned
    assert _topk(L, q=0x1002) == INVALID
    assert _topk(L, wsb=1024) == WORKSPACE
    assert _topk(L, n=(1 << 31)) == INVALID
    # per-query exclusion rows: at least ceil(n/32) words each, and a bitmap to read
    assert _topk(L, excl=0x6000, rw=-1) == INVALID
    assert _topk(L, excl=None, rw=32) == INVALID
    assert _topk(L, excl=0x6000, rw=31) == INVALID      # n = 1000 needs 32 words
    assert _topk(L, excl=0x6002, rw=32) == INVALID      # misaligned


def test_normalize_and_prepare_validation(L):
    vp = C.c_void_p
    assert L.mips_l2_normalize(None, 4, 8, F32, vp(0x1000), None) == INVALID
    assert L.mips_l2_normalize(vp(0x1000), 4, 8, FP8, vp(0x2000), None) == UNSUPPORTED
    assert L.mips_l2_normalize(vp(0x1000), -1, 8, F32, vp(0x2000), None) == INVALID
    assert L.mips_l2_normalize(vp(0x1000), 0, 8, F32, vp(0x2000), None) == OK  # nothing to do
    assert L.mips_prepare_corpus(vp(0x1000), 10, 16, 128, BF16, vp(0x2000), None, None) == INVALID
    assert L.mips_prepare_corpus(vp(0x1000), 10, 0, 128, FP8, vp(0x2000), None, None) == INVALID
    assert L.mips_prepare_corpus(vp(0x1000), 10, 0, 100, BF16, vp(0x2000), None, None) == UNSUPPORTED
    assert L.mips_prepare_corpus(vp(0x1000), 0, 0, 128, BF16, vp(0x2000), None, None) == INVALID
    assert L.mips_prepare_corpus(vp(0x1000), 10, 0, 128, BF16, vp(0x2008), None, None) == INVALID


def test_untile_inverts_the_documented_layout():
    """The test-side decoder against a hand-placed element, per dtype."""
    import numpy as np
    for dtype, E in (("f32", 4), ("bf16", 2), ("fp8", 1), ("int8", 1)):
        d, n = 128, 40
        codes = np.arange(n * d, dtype=np.int64).reshape(n, d)
        buf = np.zeros(2 * 32 * d * E, np.uint8)
        view = buf.view({4: np.uint32, 2: np.uint16, 1: np.uint8}[E])
        # place every element by the header formula, written out per element
        for row in range(n):
            for dim in range(d):
                blk, r = divmod(row, 32)
                if dtype == "f32":
                    c, rem = divmod(dim, 8)
                    t, h = divmod(rem, 2)
                elif dtype == "bf16":
                    c, rem = divmod(dim, 16)
                    h, t = divmod(rem, 8)
                elif dtype == "int8":
                    c, rem = divmod(dim, 32)
                    h, t = divmod(rem, 16)
                else:
                    j, w = divmod(dim, 64)
                    h, w2 = divmod(w, 32)
                    hi, t = divmod(w2, 16)
                    c = 2 * j + hi
                s = r + 32 * h
                off = blk * 32 * d * E + c * 1024 + s * 16 + t * E
                view[off // E] = codes[row, dim] % (1 << (8 * E))
        got = untile(buf, n, d, dtype)
        want = codes % (1 << (8 * E))
        if dtype == "f32":
            got = got.view(np.uint32)
        if dtype == "int8":
            got = got.view(np.uint8)
        assert np.array_equal(got.astype(np.int64), want)


def test_merge_rejects_bad_arguments_before_launch(L):
    vp = C.c_void_p
    offs = (C.c_int64 * 2)(0, 100)
    args = lambda **kw: dict(dict(s=vp(0x1000), i=vp(0x2000), o=C.cast(offs, vp), p=2, b=3,
                                  kin=10, kout=10, os=vp(0x3000), oi=vp(0x4000)), **kw)
    call = lambda a: L.mips_merge_topk(a["s"], a["i"], a["o"], a["p"], a["b"], a["kin"],
                                       a["kout"], a["os"], a["oi"], None)
    assert call(args(s=None)) == INVALID
    assert call(args(o=None)) == INVALID
    assert call(args(p=0)) == INVALID
    assert call(args(p=65)) == INVALID
    assert call(args(b=0)) == INVALID
    assert call(args(kin=0)) == INVALID
    assert call(args(kout=1025)) == UNSUPPORTED
    assert call(args(s=vp(0x1002))) == INVALID            # misaligned
    bad = (C.c_int64 * 2)(0, -5)
    assert call(args(o=C.cast(bad, vp))) == INVALID


def test_version_guard_fails_closed():
    import torch
    c = mips.Corpus(torch.empty(0, dtype=torch.uint8), None, 10, 16, "f32", model_version="v2")
    mips.check_version(c, "v2")
    for wrong in ("v1", None):
        with pytest.raises(mips.VersionSkew):
            mips.check_version(c, wrong)
        with pytest.raises(mips.VersionSkew):   # refused before any device work
            mips.topk(torch.empty(1, 16), c, 5, model_version=wrong)
    unversioned = mips.Corpus(torch.empty(0, dtype=torch.uint8), None, 10, 16, "f32")
    mips.check_version(unversioned, None)
    with pytest.raises(mips.VersionSkew):
        mips.check_version(unversioned, "v2")
    with pytest.raises(mips.VersionSkew):
        mips.search_shards(torch.empty(1, 16), [unversioned, c], 5, model_version="v2")


def test_topk_ranges_rejects_bad_ranges_before_launch(L):
    vp = C.c_void_p

    def call(rg, nr=None):
        arr = (C.c_int64 * max(1, len(rg)))(*rg) if rg else None
        return L.mips_topk_ranges(vp(0x1000), BF16, 4, vp(0x2000), None, BF16, 1000, 128, None, 0,
                                  None if arr is None else C.cast(arr, vp),
                                  len(rg) // 2 if nr is None else nr, 10, vp(0x3000), vp(0x4000),
                                  vp(0x5000), 1 << 30, None)
    assert call([]) == INVALID                    # no ranges
    assert call([0, 10], nr=0) == INVALID
    assert call([10, 10]) == INVALID              # empty
    assert call([5, 1001]) == INVALID             # past the corpus
    assert call([-1, 5]) == INVALID
    assert call([0, 10, 20, 15]) == INVALID       # second range inverted


def test_merge_interests_rejects_bad_arguments_before_launch(L):
    vp = C.c_void_p
    call = lambda b=2, m=4, kin=10, kout=10, s=vp(0x1000): L.mips_merge_interests(
        s, vp(0x2000), b, m, kin, kout, vp(0x3000), vp(0x4000), None)
    assert call(s=None) == INVALID
    assert call(b=0) == INVALID and call(m=0) == INVALID and call(kin=0) == INVALID
    assert call(m=4, kin=513) == UNSUPPORTED      # 2052 entries per user
    assert call(kout=1025) == UNSUPPORTED
    assert call(s=vp(0x1001)) == INVALID


def test_recall_at_k_counts_exact_ids_found():
    import numpy as np
    exact = np.array([[1, 2, 3, 4], [5, 6, -1, -1], [-1, -1, -1, -1]])
    approx = np.array([[4, 9, 2, 7, 1], [6, 5, 0, 0, 0], [3, 3, 3, 3, 3]])
    assert mips.recall_at_k(approx, exact).tolist() == [0.75, 1.0, 1.0]


def test_type_bitmap_rejects_bad_arguments_before_launch(L):
    vp = C.c_void_p
    assert L.mips_type_bitmap(None, 10, 1, None, vp(0x1000), None) == INVALID
    assert L.mips_type_bitmap(vp(0x1000), 0, 1, None, vp(0x2000), None) == INVALID
    assert L.mips_type_bitmap(vp(0x1002), 10, 1, None, vp(0x2000), None) == INVALID


def test_topk_masks_validation_and_workspace(L):
    """mips_topk_masks: argument checks before any launch, and a workspace that grows with
    the number of result sets and the candidate capacity."""
    vp = C.c_void_p
    one = L.mips_topk_masks_workspace_size(256, 10_000_000, 128, 500, BF16, BF16, 1, 0)
    four = L.mips_topk_masks_workspace_size(256, 10_000_000, 128, 500, BF16, BF16, 4, 0)
    assert 0 < one < four
    assert L.mips_topk_masks_workspace_size(256, 10_000_000, 128, 500, BF16, BF16, 5, 0) == 0
    assert L.mips_topk_masks_workspace_size(256, 10_000_000, 128, 500, BF16, BF16, 0, 0) == 0
    small = L.mips_topk_masks_workspace_size(256, 10_000_000, 128, 500, BF16, BF16, 2, 256)
    assert 0 < small < L.mips_topk_masks_workspace_size(256, 10_000_000, 128, 500, BF16, BF16, 2, 0)

    def call(masks=0x6000, nm=2, words=32, q=0x1000, ws=0x10000, wsb=1 << 30, k=10, n=1000):
        return L.mips_topk_masks(vp(q), BF16, 4, vp(0x2000), None, BF16, n, 128,
                                 None if masks is None else vp(masks), nm, words, k, vp(0x3000),
                                 vp(0x4000), vp(ws), wsb, None)
    assert call(nm=0) == INVALID
    assert call(nm=5) == UNSUPPORTED
    assert call(masks=None) == INVALID
    assert call(words=31) == INVALID         # n = 1000 needs 32 words per mask
    assert call(masks=0x6002) == INVALID     # misaligned
    assert call(q=None) == INVALID
    assert call(k=1025) == UNSUPPORTED
    assert call(wsb=1024) == WORKSPACE


def test_header_limits_match_the_binding():
    text = open(HEADER).read()
    limits = dict(re.findall(r"#define (MIPS_\w*MAX\w*) (\d+)", text))
    assert int(limits["MIPS_K_MAX"]) == mips.K_MAX
    assert int(limits["MIPS_B_MAX"]) == mips.B_MAX
    assert int(limits["MIPS_MAX_MASKS"]) == mips.MAX_MASKS


def test_batch_limit_rejected_before_launch(L):
    """More result lists than MIPS_B_MAX (one workgroup each) are refused on the host."""
    vp = C.c_void_p
    big = mips.B_MAX + 1
    assert _topk(L, b=big) == UNSUPPORTED
    assert L.mips_topk_workspace_size(big, 1000, 128, 10, BF16, BF16) == 0
    assert L.mips_topk_workspace_size_for(big, 1000, 128, 10, BF16, BF16, 100) == 0
    # four masks: b * 4 lists
    quarter = mips.B_MAX // 4 + 1
    assert L.mips_topk_masks_workspace_size(quarter, 1000, 128, 10, BF16, BF16, 4, 0) == 0
    assert L.mips_topk_masks(vp(0x1000), BF16, quarter, vp(0x2000), None, BF16, 1000, 128,
                             vp(0x6000), 4, 32, 10, vp(0x3000), vp(0x4000), vp(0x10000), 1 << 30,
                             None) == UNSUPPORTED
    offs = (C.c_int64 * 2)(0, 100)
    assert L.mips_merge_topk(vp(0x1000), vp(0x2000), C.cast(offs, vp), 2, big, 10, 10, vp(0x3000),
                             vp(0x4000), None) == UNSUPPORTED
    assert L.mips_merge_interests(vp(0x1000), vp(0x2000), big, 2, 10, 10, vp(0x3000), vp(0x4000),
                                  None) == UNSUPPORTED


def test_lattice_rows_agree_between_numpy_and_torch():
    """The deterministic pattern that large GPU inputs are built from: numpy and torch give the
    same float32 bits, including rows past 2^27."""
    import numpy as np
    from workloads import lattice_rows
    for r0, r1, d in ((0, 40, 16), ((1 << 27) - 7, (1 << 27) + 33, 16), (1000, 1003, 128)):
        a = lattice_rows(r0, r1, d)
        b = lattice_rows(r0, r1, d, "cpu").numpy()
        assert a.dtype == np.float32 and a.shape == (r1 - r0, d)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    first = lattice_rows(0, 1, 4)[0]
    want = [((12345 + j * 40503) >> 7) % 4093 - 2046 for j in range(4)]
    assert first.tolist() == [w / 256.0 for w in want]


def test_noalloc_validates_before_any_hip_call(L):
    vp = lambda x: None if x is None else C.c_void_p(x)

    def call(q=0x1000, b=4, n=1000, d=128, k=10, out_s=0x3000, out_i=0x4000, excl=None, rw=0):
        return L.mips_topk_noalloc(vp(q), BF16, b, vp(0x2000), None, BF16, n, d, vp(excl), rw, k,
                                   vp(out_s), vp(out_i), None)
    assert call(q=None) == INVALID
    assert call(out_i=None) == INVALID
    assert call(k=0) == INVALID and call(k=1025) == UNSUPPORTED
    assert call(d=48) == UNSUPPORTED
    assert call(q=0x1002) == INVALID
    assert call(excl=None, rw=40) == INVALID
    # beyond the library's scratch: the default workspace of these sizes does not fit
    assert L.mips_topk_workspace_size(1024, 100_000_000, 64, 1000, BF16, BF16) > 128 << 20
    assert call(b=1024, n=100_000_000, d=64, k=1000) == WORKSPACE
