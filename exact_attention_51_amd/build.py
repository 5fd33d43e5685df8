"""Build libfa.so (the C-ABI attention library) for gfx950 with hipcc.

Every HIP source under ``csrc/`` is compiled to an object in ``_build/`` and
linked into ``libfa.so`` next to this file.  Run as a module or call
``build()``; it always recompiles.

Flags: ``--offload-arch=gfx950`` only, ``-O3``, and packed-fp32 instruction
selection disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``):
the kernels are written with scalar float32 arithmetic throughout.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# Kernel sources never produce or test NaN on purpose: without
# -fno-honor-nans the compiler wraps every float max in a canonicalising
# v_max(x, x).  The API file (argument checks on the host) keeps full IEEE
# semantics.  MFMA results are kept in architectural VGPRs: with the default
# accumulator-register form the compiler moved the O accumulators between
# AGPRs and VGPRs on every key tile (hundreds of v_accvgpr moves per tile).
# The D = 256 forward fits the VGPR form too because it keeps its Q rows in
# LDS rather than registers.
KERNEL_FLAGS = ["-fno-honor-nans"]
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
HOST_ONLY_SOURCES = {"fa_api.hip"}


def source_flags(name: str) -> list[str]:
    if name in HOST_ONLY_SOURCES:
        return []
    return KERNEL_FLAGS + VGPR_FORM


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = source_flags(os.path.basename(src))
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libfa.so.  Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), 8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
