"""Build libcf.so (the HIP kernels and the C-ABI) for gfx950 with hipcc.

Run as ``python -m broadcast_subgraphs_amd.build`` or through
``__graft_entry__.build()``.  Compiles every time it is called.  The kernel
resource report (VGPRs, AGPRs, spills, LDS, occupancy per kernel) is written
next to the library as ``libcf.resources.txt``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcf.so")
SOURCES = ["api.hip", "stitch.hip", "gemm.hip", "unfused.hip", "spec.cpp", "auto.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed-FP32 VALU forms are disabled on purpose; the compiler still emits
    # ordinary scalar fp32 arithmetic for everything.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast",
    "-Wall",
    "-Wno-unused-result",
    "-Rpass-analysis=kernel-resource-usage",
    "-I", os.path.join(ROOT, "include"),
]
LIBS = ["-lhiprtc"]  # the runtime compiler for automatically stitched kernels


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp, *LIBS]
    proc = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    report = os.path.join(PKG, "libcf.resources.txt")
    with open(report, "w") as f:
        f.write(proc.stderr)
    if proc.returncode != 0:
        errs = "\n".join(l for l in proc.stderr.splitlines() if "error" in l or "Error" in l)
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{errs[-6000:] or proc.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
