"""Build libflashhead.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m two_stage_retrieval_amd.build        # or build() from Python
    python -m two_stage_retrieval_amd.build --no-trace   # the library only
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
OBJ_TRACE = os.path.join(ROOT, "_build", "trace")
LIB = os.path.join(PKG, "libflashhead.so")
LIB_TRACE = os.path.join(PKG, "libflashhead_trace.so")

SOURCES = ["fh_api.hip", "fh_stage1.hip", "fh_decode_b1_adapt.hip", "fh_rowdot.hip",
           "fh_select.hip",
           "fh_prepare.hip", "fh_batched.hip", "fh_mc.hip",
           "fh_kmeans.hip", "fh_host.cpp"]

# Packed-fp32 instructions are disabled for all device code.  Leading scalar
# kernel arguments (up to 8 dwords) are preloaded into scalar registers by
# the dispatcher, so a kernel's first requests need not wait for its
# argument loads (kernels that take one argument struct are unaffected).
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=8",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm toolchain required)")
    return exe


def _compile(src: str, trace: bool = False) -> str:
    obj_dir = OBJ_TRACE if trace else OBJ
    out = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *(["-DFH_TRACE"] if trace else []), "-c",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


def build(verbose: bool = False, trace: bool = True) -> str:
    """Compiles libflashhead.so and, with trace, its measurement build
    libflashhead_trace.so (the same sources with the timeline hooks of
    fh_trace.h compiled in).  Returns the library's path."""
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(OBJ_TRACE, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = [(s, False) for s in srcs] + ([(s, True) for s in srcs] if trace else [])
    with cf.ThreadPoolExecutor(max_workers=min(16, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    for lib, variant in ((LIB, False), (LIB_TRACE, True)):
        if variant and not trace:
            continue
        sel = [o for o, (_, t) in zip(objs, jobs) if t == variant]
        tmp = lib + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *sel, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


if __name__ == "__main__":
    build(verbose=True, trace="--no-trace" not in sys.argv)
    sys.exit(0)
