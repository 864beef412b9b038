"""Build libpsgd.so (host plan code + gfx950 HIP kernels of the PowerSGD, rTop-k and
Spectral-ATOMO compressors) in-tree with hipcc.

    python -m distributed_sgd_gradient_ef_amd.build

The library is written next to this file; the Python binding loads it from there.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libpsgd.so")
SOURCES = [os.path.join(HERE, "csrc", name) for name in ("plan.cpp", "kernels.hip", "rtopk.hip", "atomo.hip")]
INCLUDE = [os.path.join(ROOT, "include"), os.path.join(HERE, "csrc")]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions
# (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32); ordinary fp32 code is used instead.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpsgd)")


def build(verbose: bool = False) -> str:
    """Compile every source into LIB_PATH (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *[f"-I{d}" for d in INCLUDE], *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
