"""The profiling hook mips_set_timing_events: the main score kernel's dispatch records the two
caller-owned hipEvents around that kernel on the call's stream. Checked through the C ABI: the
bracketed span is positive and inside the whole call's span, the results are bitwise those of
a call without the hook, and clearing the hook stops the recording."""
import ctypes as C

import numpy as np
import pytest
import torch

import exact_inner_product_amd as mips
from workloads import WORKLOADS

pytestmark = pytest.mark.gpu


class _HipEvents:
    def __init__(self):
        self.L = C.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.L.hipEventSynchronize.argtypes = [C.c_void_p]
        self.L.hipEventQuery.argtypes = [C.c_void_p]
        self.L.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        ev = C.c_void_p()
        assert self.L.hipEventCreate(C.byref(ev)) == 0
        return ev

    def elapsed_ms(self, a, b):
        assert self.L.hipEventSynchronize(b) == 0
        ms = C.c_float()
        rc = self.L.hipEventElapsedTime(C.byref(ms), a, b)
        return ms.value if rc == 0 else None


@pytest.mark.parametrize("n", [300_000, 2_000])  # sampled passes; the dense pass
def test_timing_events_bracket_the_main_pass_and_change_nothing(n):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    dev = torch.device("cuda:0")
    w = WORKLOADS["bf16_n1m_d128_b16"].replace(n=n, b=40, k=100, seed=31)
    corpus = mips.prepare_corpus(torch.from_numpy(w.corpus()).to(dev), "bf16")
    q = mips.l2_normalize(torch.from_numpy(w.queries()).to(dev), "bf16")
    s0, i0 = mips.topk(q, corpus, w.k)
    torch.cuda.synchronize()

    hip = _HipEvents()
    before, after = hip.create(), hip.create()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mips.set_timing_events(before, after)
    try:
        t0.record()
        s1, i1 = mips.topk(q, corpus, w.k)
        t1.record()
    finally:
        mips.set_timing_events(None, None)
    torch.cuda.synchronize()
    main_ms = hip.elapsed_ms(before, after)
    call_ms = t0.elapsed_time(t1)
    print(f"n={n}: main kernel {main_ms * 1e3:.1f} us of a {call_ms * 1e3:.1f} us call")
    assert main_ms is not None and 0.0 < main_ms <= call_ms
    assert np.array_equal(s0.cpu().numpy().view(np.uint32), s1.cpu().numpy().view(np.uint32))
    assert np.array_equal(i0.cpu().numpy(), i1.cpu().numpy())

    # cleared: a later call records nothing, so the pair keeps the span measured above
    s2, i2 = mips.topk(q, corpus, w.k)
    torch.cuda.synchronize()
    assert hip.elapsed_ms(before, after) == pytest.approx(main_ms)
    assert np.array_equal(i0.cpu().numpy(), i2.cpu().numpy())
    hip.L.hipEventDestroy(before)
    hip.L.hipEventDestroy(after)
