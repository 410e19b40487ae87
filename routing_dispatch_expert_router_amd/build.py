"""Build libmoe.so (gfx950 code objects + C-ABI host code) in-tree with hipcc.

    python routing_dispatch_expert_router_amd/build.py [-v]

(run it by path: importing the package loads the library it builds)

Every source is compiled on each call (object files go to _build/ at the repo
root); the shared library is written next to this file and replaced atomically.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are disabled for every device pass.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]
SOURCES = ["route.hip", "dispatch.hip", "gemm.hip", "mlp.hip", "combine.hip", "backward.hip", "moe_api.cpp"]


def _compile(src, obj, verbose):
    cmd = [HIPCC, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; that warning is expected
    noise = [l for l in r.stderr.splitlines() if l.strip() and "packed-fp32-ops" not in l]
    if verbose and noise:
        print("\n".join(noise))
    return obj


def build(verbose=False):
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(SOURCES, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # a kernel template whose host-side instantiation failed leaves its launch
    # stub undefined; refuse such a library instead of failing at load time
    nm = subprocess.run(["nm", "-DC", "--undefined-only", tmp], capture_output=True, text=True)
    bad = [l.strip() for l in nm.stdout.splitlines() if "moe::" in l]
    if bad:
        os.remove(tmp)
        raise RuntimeError("libmoe.so has undefined library symbols:\n" + "\n".join(bad[:20]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
