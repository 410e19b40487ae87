"""The library's host code under AddressSanitizer (CPU only, no GPU needed).

tests/asan/build_asan.py builds libmoe with -fsanitize=address on every host
pass (device code as usual); tests/asan/harness.cpp, built with the same
sanitizer, drives the configuration checks, the size helpers and every entry
point's argument checks.  Any host memory error aborts the harness with an
AddressSanitizer report.  Leak checking is off: the HIP runtime's own
allocations at exit are not this library's.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(CLANG) and shutil.which("nm")), reason="ROCm clang not installed")
def test_host_code_under_asan(tmp_path):
    from tests.asan import build_asan
    lib = build_asan.build()
    exe = str(tmp_path / "harness")
    subprocess.run([CLANG, "-std=c++17", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    os.path.join(HERE, "asan", "harness.cpp"), lib, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath," + os.path.dirname(lib) + ":/opt/rocm/lib", "-o", exe], check=True,
                   capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr[-2000:])
