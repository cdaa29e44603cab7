"""Build libcf.so (the HIP kernels and the C-ABI) for gfx950 with hipcc.

Run as ``python -m broadcast_subgraphs_amd.build`` or through
``__graft_entry__.build()``.  Compiles every time it is called: each source
into its own object under ``_build/`` (the sources compile in parallel), then
one link.  The kernel resource report (VGPRs, AGPRs, spills, LDS, occupancy
per kernel) is written next to the library as ``libcf.resources.txt``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcf.so")
SOURCES = ["api.hip", "stitch.hip", "gemm.hip", "unfused.hip", "spec.cpp", "auto.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
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


def _compile(src: str) -> tuple[str, subprocess.CompletedProcess]:
    obj = os.path.join(OBJ, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    return obj, subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    report = os.path.join(PKG, "libcf.resources.txt")
    with open(report, "w") as f:
        for _, proc in results:
            f.write(proc.stderr)
    for src, (_, proc) in zip(SOURCES, results):
        if proc.returncode != 0:
            errs = "\n".join(l for l in proc.stderr.splitlines() if "error" in l or "Error" in l)
            raise RuntimeError(f"hipcc failed on {src} ({proc.returncode}):\n{errs[-6000:] or proc.stderr[-6000:]}")
    tmp = LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in results], "-o", tmp, *LIBS]
    proc = subprocess.run(link, cwd=CSRC, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed ({proc.returncode}):\n{proc.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
