"""The host side of the library (argument validation, planning, workspace
layout) built with AddressSanitizer by g++ and run under the whole host API
test file (``tests/test_api.py``), on the CPU.  The kernels are not part of
this build: its launch helpers are stubs (``tests/asan_launch_stubs.cpp``),
which no host test reaches."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_bwd_amd", "csrc")


def _libasan():
    gxx = shutil.which("g++")
    if gxx is None:
        return None, None
    path = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return gxx, (path if os.path.isabs(path) and os.path.exists(path) else None)


def test_host_library_under_address_sanitizer(tmp_path):
    gxx, libasan = _libasan()
    if libasan is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("g++ with libasan and the HIP runtime are needed")
    lib = str(tmp_path / "libbsa_bwd_asan.so")
    build = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address", "-fno-omit-frame-pointer",
             "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             os.path.join(CSRC, "bsa_api.cpp"), os.path.join(ROOT, "tests", "asan_launch_stubs.cpp"),
             "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", lib]
    r = subprocess.run(build, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, BSA_LIBRARY=lib, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_api.py"), os.path.join(ROOT, "tests", "test_api_fp8.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
