"""Build the library with AddressSanitizer on its host code (the device code is built as usual):
_build/asan/libmoe_asan.so, for the host-side argument-checking harness (CPU only).

Every host pass gets -fsanitize=address through -Xarch_host, so no device code is instrumented.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "routing_dispatch_expert_router_amd")
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(ROOT, "_build", "asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["route.hip", "dispatch.hip", "gemm.hip", "mlp.hip", "combine.hip", "backward.hip", "moe_api.cpp"]
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"] + HOST_ASAN


def _compile(src):
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build():
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    lib = os.path.join(OUT, "libmoe_asan.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_ASAN, "-o", lib, *objs],
                       capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build())
