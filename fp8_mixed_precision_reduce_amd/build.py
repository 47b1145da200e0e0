"""Build libfp8lin.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Each translation unit is compiled separately (in parallel) and the objects are
linked into fp8_mixed_precision_reduce_amd/libfp8lin.so.  Flags:
  --offload-arch=gfx950           MI355X only
  -O3 -std=c++17 -fPIC
  -ffp-contract=off               every a*b+c stays two rounded operations unless
                                  the source asks for an FMA (bit-exact casts)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                  no packed-fp32 VALU instructions
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfp8lin.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["elementwise.hip", "cast_transpose.hip", "gemm.hip", "training.hip", "attention.hip", "api.cpp"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _compile(src, verbose):
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise and verbose:
        print("\n".join(noise), flush=True)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
