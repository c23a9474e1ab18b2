"""Build libzq.so (the HIP kernels and C ABI) in-tree for gfx950.

    python -m int4_quantized_transformer_amd.build

Compiles every ``csrc/*.hip`` with hipcc and links ``libzq.so`` next to this
file.  Flags that matter for correctness:
  * ``-fhip-fp32-correctly-rounded-divide-sqrt`` and no fast-math: the
    quantizer's fp32 division must be IEEE round-to-nearest so that codes
    match a plain CPU evaluation bit for bit;
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32
    instructions are generated.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libzq.so")
ARCH = os.environ.get("ZQ_OFFLOAD_ARCH", "gfx950")


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip"))


def _compile(src, verbose):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + COMMON + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if err and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
