"""The C ABI from a plain C99 program (tests/c_abi_example.c): it compiles and links
against include/mips.h and libmips.so with gcc alone (CPU), and on a GPU it builds an
index, searches it and checks the result against its own brute-force scan."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_example.c")
LIBDIR = os.path.join(ROOT, "exact_inner_product_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIBDIR, "libmips.so")):
        pytest.skip("libmips.so not built")
    exe = str(tmp_path / "c_abi_example")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-O1", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", SRC, "-o", exe, f"-L{LIBDIR}", "-lmips",
           f"-L{ROCM}/lib", "-lamdhip64", "-lm", f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{ROCM}/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def test_c_example_compiles_and_links(tmp_path):
    _build(tmp_path)


@pytest.mark.gpu
def test_c_example_runs(tmp_path):
    exe = _build(tmp_path)
    print("c abi example: n=5000 d=64 b=9 k=25 f32", flush=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c abi ok" in res.stdout
