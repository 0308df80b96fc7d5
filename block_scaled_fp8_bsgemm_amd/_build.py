"""Build libbsgemm.so (the HIP kernels + C ABI) for gfx950, in-tree.

``python -m block_scaled_fp8_bsgemm_amd._build`` compiles every source under
``csrc/`` with hipcc into ``block_scaled_fp8_bsgemm_amd/libbsgemm.so``.  It
cross-compiles on a machine without a GPU.  Flags:

  --offload-arch=gfx950          MI355X only, no other targets
  -O3, no fast-math              IEEE fp32/fp64 division and denormals are
                                 part of the quantizer's exactness argument
  -packed-fp32-ops disabled      packed fp32 VALU forms are kept out of the
                                 generated code
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbsgemm.so")

SOURCES = ["gemm.hip", "stream.hip", "abi.cpp"]
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libbsgemm)")


def build(verbose=False, extra_flags=()):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags) + ["-I", INCLUDE, "-I", CSRC] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and "(ignoring feature)" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
