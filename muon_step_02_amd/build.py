"""Build libmuon.so (the HIP library behind include/muon.h) in-tree for gfx950.

``python -m muon_step_02_amd.build`` or ``build()`` compiles every source in
csrc/ with hipcc and links muon_step_02_amd/libmuon.so.  Always rebuilds.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmuon.so")

SOURCES = ["api.hip", "plan.cpp", "elementwise.hip", "gemm_bf16.hip", "gemm_f32.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-strict-aliasing",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
    # never let the compiler form packed fp32 adds/muls/fmas
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src):
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
