"""Build libreplayssm.so in-tree with hipcc for gfx950.

Usage: python -m linear_recurrence_amd._build   (or __graft_entry__.build()).
Each HIP source compiles to an object in parallel (the host-only metadata
helpers with the host C++ compiler); the objects link into
``linear_recurrence_amd/libreplayssm.so``.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libreplayssm.so")
SOURCES = ("mamba2_decode.hip", "mamba2_sr.hip", "mamba2_small.hip", "gdn_decode.hip",
           "gdn_spec.hip", "metadata.cpp")
CXX = os.environ.get("CXX", "g++")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-mcode-object-version=5",
    # keep the compiler away from packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src):
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    if src.endswith(".cpp"):  # host-only code
        inc = ["-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
               "-D__HIP_PLATFORM_AMD__"]
        cmd = [CXX, "-O2", "-std=c++17", "-fPIC", "-Wall", *inc, "-c",
               os.path.join(CSRC, src), "-o", out]
    else:
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"compile failed for {src}:\n{r.stderr}")
    return out


def build(verbose=True):
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
