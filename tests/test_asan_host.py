"""The library's host code (argument validation, planning, workspace
arithmetic: api.hip) built with AddressSanitizer on the host side only,
linked with the ordinary kernel objects, and driven on the CPU by
tests/c/abi_validation.c (every call fails validation or only sizes a
workspace, so no device is needed). An out-of-bounds access, use after free
or similar memory error in that host code aborts the program."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "lm_head_gemm_amd")
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.timeout(600)
def test_host_code_under_address_sanitizer(tmp_path):
    from lm_head_gemm_amd import build
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.hip.o")))
    others = [o for o in objs if os.path.basename(o) != "api.hip.o"]
    if not others:
        pytest.fail("kernel objects not built (python -m lm_head_gemm_amd.build)")
    api_o = str(tmp_path / "api_asan.o")
    # host pass instrumented; the device pass of the same file is left alone
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in build.HIP_FLAGS if f != "-O3"] + ["-O1", "-g"]
    cmd = [build.hipcc(), *flags, *host_asan, "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    lib = str(tmp_path / "libflashsample.so")
    r = subprocess.run([build.hipcc(), "-shared", "-fPIC", f"--offload-arch={build.ARCH}", api_o, *others,
                        "-o", lib], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "abi_validation")
    r = subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
                        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        os.path.join(ROOT, "tests", "c", "abi_validation.c"), "-o", exe, "-L", str(tmp_path),
                        "-lflashsample", "-L", "/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{tmp_path}",
                        "-Wl,-rpath,/opt/rocm/lib", "-lm"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr
    print(r.stdout.strip())
