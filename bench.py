"""Benchmark of exhaustive inner-product top-K (mips_topk) on one MI355X.

A step is one mips_topk call over a batch that is already resident in HBM: query prep,
sampled threshold, the fused MFMA score/filter pass and the final merge. Default workload:
N=10,000,000 x D=128 bf16 corpus (clustered/Zipf, 16384 clusters), B=256 queries, K=500,
5% of ids excluded. Prints one JSON line.

    python bench.py [--gpus 1] [--steps 40] [--warmup 3] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_kernel_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_inner_product_amd", "csrc", f)
                  for f in ("score.h", "score_api.h", "score_inst.hip", "common.h")]
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "int8": 5033.2, "f32": 157.3}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """hipEvents through the HIP runtime, for timing on the stream the kernels run on."""

    def __init__(self):
        self.L = C.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.L.hipEventSynchronize.argtypes = [C.c_void_p]
        self.L.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        ev = C.c_void_p()
        assert self.L.hipEventCreate(C.byref(ev)) == 0
        return ev

    def elapsed_ms(self, a, b):
        assert self.L.hipEventSynchronize(b) == 0
        ms = C.c_float()
        assert self.L.hipEventElapsedTime(C.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, ev):
        self.L.hipEventDestroy(ev)


def kernel_source_hash():
    """Hash of the main score pass's sources with comments and blank lines dropped, so that a
    counter summary stays valid across edits that do not change the code."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        for line in open(f, encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per main-pass launch from the committed counter summary, if it was taken
    on the current kernel source and this workload; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if fields.get("workload") != workload:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, dev, gib):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 copies of {n * 4} bytes")


def copy_probe_gbs(torch, dev, gib=1.0, reps=5):
    """Measured HBM bandwidth of a plain device-to-device copy of `gib` GiB (bytes read +
    bytes written per second), a practical ceiling reported beside the published peak."""
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2.0 * n * 4 / (ms / 1e3) / 1e9


def build_gpu_inputs(w, dev, torch, mips):
    """Raw corpus chunks -> device -> mips_prepare_corpus; queries -> mips_l2_normalize."""
    corpus = mips.empty_corpus(w.n, w.d, w.corpus_dtype, dev)
    t_prep = 0.0
    nbytes_in = 0
    nchunks = 0
    for r0, blk in w.corpus_chunks():
        nchunks += 1
        if nchunks % 16 == 0:
            log(f"index build: {r0 + blk.shape[0]} of {w.n} rows")
        x = torch.from_numpy(blk).to(dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        mips.prepare_rows(corpus, x, r0)
        torch.cuda.synchronize()
        t_prep += time.perf_counter() - t0
        nbytes_in += blk.nbytes
        del x
    q = mips.l2_normalize(torch.from_numpy(w.queries()).to(dev), w.query_dtype)
    bm = w.exclude_bitmap()
    excl = None if bm is None else torch.from_numpy(bm.view(np.int32)).to(dev)
    torch.cuda.synchronize()
    out_bytes = corpus.packed.numel() + (0 if corpus.row_scale is None else corpus.row_scale.numel() * 4)
    return corpus, q, excl, (nbytes_in + out_bytes) / t_prep / 1e9


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_queries):
    """The oracle as it stands (int8 index: its quantised scoring branch), on the first
    `budget_queries` queries of the same workload against the whole corpus. The rate in
    scores/s is measured on that sample; the time of the whole batch at that rate is an
    extrapolation and is labelled as one."""
    import oracle
    t0 = time.perf_counter()
    codes, scale = oracle.prepare_chunks(w.corpus_chunks(), w.n, w.d, w.corpus_dtype)
    q_or, _ = oracle.prepare(w.queries()[:budget_queries], w.query_dtype)
    bm = w.exclude_bitmap()
    log(f"oracle inputs ready in {time.perf_counter() - t0:.1f}s")
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    if w.corpus_dtype == "int8":
        oracle.topk_int8(q_or, w.query_dtype, codes, w.k, scale, exclude=bm, threads=threads)
    else:
        oracle.topk(q_or, w.query_dtype, codes, w.corpus_dtype, w.k, row_scale=scale,
                    exclude=bm, threads=threads)
    dt = time.perf_counter() - t0
    used = min(threads, budget_queries)
    return {"value": budget_queries * w.n / dt, "unit": "scores/s",
            "cores": used, "kind": "oracle",
            "sample": f"first {budget_queries} of {w.b} queries against the full corpus "
                      f"(n={w.n}, d={w.d}, k={w.k}), {dt:.1f}s; exact fp64 dot products and "
                      f"a full sort per query; the whole batch of {w.b} would take "
                      f"{dt * w.b / budget_queries:.0f}s at this rate (extrapolated)",
            "cpu_model": cpu_model(), "threads": used,
            "batch_seconds_extrapolated": dt * w.b / budget_queries}


def bench_masks(args, w, corpus, q, excl, torch, mips, dev):
    """One multi-mask pass against T separate calls, each with one mask as its bitmap; the
    same synthetic masks, inputs resident, the same step count for both."""
    import numpy as np
    from workloads import typed_masks
    t = args.masks
    if not 1 <= t <= 4:
        log("--masks takes 1 to 4")
        sys.exit(2)
    base = None if excl is None else excl.cpu().numpy().view(np.uint32)
    rows = typed_masks(w.n, base)[:t]
    masks = torch.from_numpy(rows.view(np.int32)).to(dev)
    wsm = mips.empty_workspace(mips.masks_workspace_size(w.b, w.n, w.d, w.k, w.query_dtype,
                                                         w.corpus_dtype, t), dev)
    ws1 = mips.empty_workspace(mips.workspace_size(w.b, w.n, w.d, w.k, w.query_dtype,
                                                   w.corpus_dtype), dev)

    def one_pass():
        mips.topk_masks(q, corpus, masks, w.k, workspace=wsm)

    def separate():
        for r in range(t):
            mips.topk(q, corpus, w.k, masks[r], workspace=ws1)

    def timed(f):
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            f()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    ms_pass = timed(one_pass)
    ms_sep = timed(separate)
    log(f"{t} masks: one pass {ms_pass:.3f} ms, {t} separate calls {ms_sep:.3f} ms")
    print(json.dumps({
        "metric": "query-item scores/s (exhaustive inner-product top-K, multi-mask pass)",
        "value": w.b * w.n / (ms_pass / 1e3), "unit": "scores/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_pass,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.corpus_dtype, "data": "synthetic",
        "config": {"workload": w.name, "masks": t, "n": w.n, "d": w.d, "b": w.b, "k": w.k},
        "separate_calls_ms": ms_sep, "speedup_vs_separate": ms_sep / ms_pass,
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-queries", type=int, default=0,
                    help="queries in the CPU-baseline sample (default: twice the host "
                         "threads, at most 32, at most the batch)")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="MiB of scratch read before every timed call (0: none)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="first run a plain device copy of GIB GiB (counter calibration)")
    ap.add_argument("--masks", type=int, default=0, metavar="T",
                    help="time a T-mask pass (mips_topk_masks, 1 <= T <= 4, the item-type "
                         "masks of workloads.typed_masks) beside T separate mips_topk calls")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; use --gpus 1"}))
        sys.exit(2)

    import torch

    import exact_inner_product_amd as mips
    from workloads import HEADLINE, WORKLOADS

    w = WORKLOADS[args.workload or HEADLINE]
    dev = torch.device("cuda:0")
    if args.copy_calibration > 0:
        copy_calibration(torch, dev, args.copy_calibration)
    log(f"workload {w.name}: n={w.n} d={w.d} b={w.b} k={w.k} {w.corpus_dtype}")
    t0 = time.perf_counter()
    corpus, q, excl, prep_gbs = build_gpu_inputs(w, dev, torch, mips)
    log(f"inputs resident in HBM after {time.perf_counter() - t0:.1f}s; prepare {prep_gbs:.0f} GB/s")

    if args.masks:
        return bench_masks(args, w, corpus, q, excl, torch, mips, dev)

    wsb = mips.workspace_size(w.b, w.n, w.d, w.k, w.query_dtype, w.corpus_dtype)
    ws = mips.empty_workspace(wsb, dev)
    scores = torch.empty((w.b, w.k), dtype=torch.float32, device=dev)
    ids = torch.empty((w.b, w.k), dtype=torch.int32, device=dev)
    # read before every timed call (outside its events) so that no call finds the corpus in
    # the 256 MB last-level cache; written once here, so the cache holds no dirty lines whose
    # write-back would compete with the call's reads
    flush = torch.ones(args.flush_mib << 18, dtype=torch.float32, device=dev) \
        if args.flush_mib > 0 else None
    flush_out = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        mips.topk(q, corpus, w.k, excl, workspace=ws, out=(scores, ids))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    # The main-pass duration comes from events the kernel's dispatch records; those events
    # add a dispatch gap of several microseconds on each side of the kernel, so only every
    # other timed call carries them, and the call time reported as the metric is the median
    # of the calls without (both kinds do the same work).
    timed = [i % 2 == 1 for i in range(args.steps)] if args.steps > 1 else [True]
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            torch.sum(flush, dim=0, out=flush_out)
        if timed[i]:
            mips.set_timing_events(pairs[i][0], pairs[i][1])
        calls[i][0].record()
        step()
        calls[i][1].record()
        mips.set_timing_events(None, None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    main_ms = [ev.elapsed_ms(a, b) for (a, b), t in zip(pairs, timed) if t]
    call_all = [a.elapsed_time(b) for a, b in calls]
    call_ms = [c for c, t in zip(call_all, timed) if not t] or call_all
    call_ev_ms = [c for c, t in zip(call_all, timed) if t]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    log(f"timed {args.steps} steps in {wall:.3f}s (with a {args.flush_mib} MiB read before "
        f"each); per call: median {np.median(call_ms):.4f} ms, min {min(call_ms):.4f} ms")

    # back to back with no flush: the rate of a stream of calls on one index (labelled extra)
    torch.cuda.synchronize()
    tb = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - tb) / args.steps * 1e3

    ms_per_step = float(np.median(call_ms))
    scores_per_s = w.b * w.n / (ms_per_step / 1e3)
    E = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1}[w.corpus_dtype]
    # Algorithmic bytes of the main score pass: every packed corpus row once (plus its
    # fp8 or int8 scale), the exclusion bitmap and the queries.
    alg_bytes = w.n * w.d * E + (4 * w.n if w.corpus_dtype in ("fp8", "int8") else 0)
    alg_bytes += (w.n / 8 if w.exclude_frac > 0 else 0) + w.b * w.d * E
    flops = 2.0 * w.b * w.n * w.d
    main_avg = float(np.mean(main_ms)) / 1e3
    achieved_gbs = alg_bytes / main_avg / 1e9
    achieved_tflops = flops / main_avg / 1e12
    t_hbm = alg_bytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = flops / (PEAK_TFLOPS[w.corpus_dtype] * 1e12)
    call_s = ms_per_step / 1e3
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved_gbs / PEAK_HBM_GBS}
        call_frac = alg_bytes / call_s / 1e9 / PEAK_HBM_GBS
    else:
        roof = {"bound": "mfma", "achieved": achieved_tflops, "peak": PEAK_TFLOPS[w.corpus_dtype],
                "unit": "TFLOP/s", "frac": achieved_tflops / PEAK_TFLOPS[w.corpus_dtype]}
        call_frac = flops / call_s / 1e12 / PEAK_TFLOPS[w.corpus_dtype]
    roof["traffic"] = measured_traffic(w.name)
    roof["kernel"] = "score_kernel (main pass)"
    roof["kernel_avg_us"] = main_avg * 1e6
    roof["kernel_median_us"] = float(np.median(main_ms)) * 1e3
    roof["algorithmic_bytes"] = alg_bytes
    roof["mfma_frac"] = achieved_tflops / PEAK_TFLOPS[w.corpus_dtype]
    # the same roofline for the whole call (every kernel of mips_topk, median of the timed
    # calls): what the metric measures
    roof["call_frac"] = call_frac
    roof["call_median_ms"] = ms_per_step
    roof["call_min_ms"] = float(min(call_ms))
    # measured after the timed region: the HBM rate of a plain 1 GiB device copy
    copy_gbs = copy_probe_gbs(torch, dev)
    roof["copy_gbs"] = copy_gbs
    roof["hbm_frac_of_copy"] = achieved_gbs / copy_gbs
    log(f"device copy probe: {copy_gbs:.0f} GB/s; main pass at {achieved_gbs / copy_gbs:.3f} of it")

    result = {
        "metric": "query-item scores/s (exhaustive inner-product top-K)",
        "value": scores_per_s,
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.corpus_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "d": w.d, "b": w.b, "k": w.k,
                   "corpus_dtype": w.corpus_dtype, "query_dtype": w.query_dtype,
                   "exclude_frac": w.exclude_frac, "clusters": w.clusters},
        "queries_per_s": w.b / (ms_per_step / 1e3),
        "timing": {"per_call": "HIP events around each mips_topk call on its stream, after "
                               f"reading {args.flush_mib} MiB of scratch (untimed); "
                               "value and ms_per_step use the median of the calls that do "
                               "not also time their main pass",
                   "median_ms": ms_per_step, "min_ms": float(min(call_ms)),
                   "calls": len(call_ms),
                   "median_ms_of_calls_timing_the_main_pass": float(np.median(call_ev_ms)),
                   "wall_ms_per_step_incl_flush": wall / args.steps * 1e3,
                   "back_to_back_unflushed_ms": warm_ms},
        "prepare_gbs": prep_gbs,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        nq = args.cpu_queries or min(w.b, 32, 2 * max(1, len(os.sched_getaffinity(0))))
        log(f"cpu baseline: oracle on {nq} queries")
        result["cpu_baseline"] = cpu_baseline(w, nq)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
