"""The boundary from plain C: tests/c/sample_from_c.c includes only
include/flashsample.h and the HIP runtime, links libflashsample.so, and
drives the fused (row-major and tiled) and unfused entry points. On the CPU
it is compiled and linked as C11 with warnings as errors; on the GPU it runs
as a child process and its tokens are checked against the oracle."""
import os
import subprocess

import numpy as np
import pytest

from tests._util import check_parity

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "sample_from_c.c")
LIBDIR = os.path.join(ROOT, "lm_head_gemm_amd")


def _build(out):
    if not os.path.exists(os.path.join(LIBDIR, "libflashsample.so")):
        pytest.fail("libflashsample.so not built (python -m lm_head_gemm_amd.build)")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", SRC, "-o", str(out),
           "-L", LIBDIR, "-lflashsample", "-L", "/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr


def test_c_program_compiles_and_links(tmp_path):
    _build(tmp_path / "sample_from_c")


@pytest.mark.gpu
def test_c_program_samples_like_the_oracle(tmp_path):
    exe = tmp_path / "sample_from_c"
    _build(exe)
    B, D, V, T, seed, step = 20, 512, 3001, 0.8, 5, 2
    r = subprocess.run([str(exe), str(tmp_path), str(B), str(D), str(V), str(T), str(seed), str(step)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    out = {line.split()[0]: line.split()[1:] for line in r.stdout.splitlines()}
    assert out["error"] == ["FS_ERR_INVALID_ARGUMENT"]
    H = np.fromfile(tmp_path / "H.bin", dtype=np.uint16).reshape(B, D)
    W = np.fromfile(tmp_path / "W.bin", dtype=np.uint16).reshape(V, D)
    rows = np.array(out["rows"], dtype=np.int64)
    assert np.array_equal(rows, np.array(out["tiled"], dtype=np.int64))
    for name in ("rows", "unfused"):
        check_parity(H, W, T, seed, step, np.arange(B), np.array(out[name], dtype=np.int64))
