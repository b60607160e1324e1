"""Build step of libmips.so: hipcc for gfx950, in-tree.

The score pass is compiled once per (corpus dtype, width) pair from score_inst.hip, each
into its own object, in parallel; the objects are then linked into libmips.so next to this
file.

Usage: python -m exact_inner_product_amd.build [-v]   (or call build()).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmips.so")
SOURCES = ["api.hip", "normalize.hip", "topk.hip", "merge.hip", "noalloc.hip"]

# (dtype macro, width) pairs of the score pass; must match corpus_d_supported in host.h
SCORE_UNITS = ([("MIPS_F32", d) for d in (16, 32, 64, 128)] +
               [("MIPS_BF16", d) for d in (16, 32, 64, 128, 256)] +
               [("MIPS_FP8_E4M3", d) for d in (64, 128, 256)] +
               [("MIPS_INT8", d) for d in (32, 64, 128, 256)])

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # no packed-fp32 VALU instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    # MFMA accumulators in VGPRs, where the top-K epilogue reads them; operands that only
    # the matrix pipe reads may then live in AGPRs.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def _jobs():
    n = os.environ.get("MAX_JOBS") or os.cpu_count() or 4
    return max(1, min(16, int(n)))


def build(verbose: bool = False) -> str:
    if os.path.isdir(OBJ_DIR):
        shutil.rmtree(OBJ_DIR)
    os.makedirs(OBJ_DIR)
    units = [(os.path.join(CSRC, s), [], os.path.join(OBJ_DIR, s.replace(".hip", ".o")))
             for s in SOURCES]
    for ct, d in SCORE_UNITS:
        obj = os.path.join(OBJ_DIR, f"score_{ct.split('_', 1)[1].lower()}_d{d}.o")
        units.append((os.path.join(CSRC, "score_inst.hip"), [f"-DMIPS_CT={ct}", f"-DMIPS_D={d}"], obj))

    def compile_one(unit):
        src, defs, obj = unit
        cmd = [HIPCC, *FLAGS, *defs, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src} {defs}:\n{res.stderr}")
        return obj

    with cf.ThreadPoolExecutor(_jobs()) as ex:
        objs = list(ex.map(compile_one, units))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
