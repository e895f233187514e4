"""Builds libzero_mi355x.so in-tree with hipcc for gfx950.

Translation units: the host planner, checkpoint and offload code (C++) and
the HIP device path.  All HIP code is compiled without packed-fp32
instructions and without denormal flushing.

A second library, libzero_mi355x_capped.so, is the same code with the
per-launch block cap lowered to 64 blocks, so that tests reach the
multi-launch and multi-round paths (taken above about 17e9 elements with
the real cap) on small inputs.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzero_mi355x.so")
CAPPED_LIB = os.path.join(PKG, "libzero_mi355x_capped.so")
CAPPED_BLOCKS = 64
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-flush-denormals-to-zero", "-Wno-unused-command-line-argument"]

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST = [f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__=1"]  # HIP runtime API from host C++

SOURCES = ["zero_host.cpp", "zero_ckpt.cpp", "zero_offload.cpp", "zero_kernels.hip", "zero_adam.hip"]
# the host AdamW of the offload path: OpenMP threads, vectorisable sqrt, and the
# exact operation sequence of the device kernel (no contraction)
EXTRA = {"zero_offload.cpp": ["-fopenmp", "-fno-math-errno", "-ffp-contract=off"]}
LINK = ["-fopenmp", f"-Wl,-rpath,{ROCM}/lib/llvm/lib"]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def _link(objs, out):
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *LINK, "-o", tmp])
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    """Compile every source and link both libraries (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD_DIR, src + ".o")
        if src.endswith(".hip"):
            _run([HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", path, "-o", obj])
        else:
            _run([HIPCC, *COMMON, *HOST, *EXTRA.get(src, []), "-x", "c++", "-c", path, "-o",
                  obj])
        objs.append(obj)
    _link(objs, LIB)
    capped = []
    for src, obj in zip(SOURCES, objs):
        if src.endswith(".hip"):
            obj = os.path.join(BUILD_DIR, src + ".capped.o")
            _run([HIPCC, *COMMON, *DEVICE, f"-DZERO_MAX_LAUNCH_BLOCKS={CAPPED_BLOCKS}", "-x",
                  "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        capped.append(obj)
    _link(capped, CAPPED_LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
