"""Build of the gfx950 shared library libbefmoe.so (hipcc, in-tree).

All HIP sources are compiled for gfx950 only, with IEEE fp32 division and
square root (the hipcc default, stated explicitly) and without fast-math or
denormal flushing, and with packed-fp32 instruction selection turned off.
MFMA results are kept in ordinary VGPRs (-amdgpu-mfma-vgpr-form): the
grouped GEMM folds every MFMA result into its accumulators with VALU FMAs,
which cannot read AGPRs.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SO = os.path.join(PKG, "libbefmoe.so")
SOURCES = ["moe_api.hip", "actq.hip", "route.hip", "permute.hip", "gemv.hip", "gemm.hip",
           "combine.hip", "decode.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=fast",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False, extra: list[str] | None = None, out: str | None = None) -> str:
    """Compile each source to an object (in parallel), then link the library."""
    from concurrent.futures import ThreadPoolExecutor
    out = out or SO
    objdir = os.path.join(ROOT, "_build", os.path.basename(out) + ".objs")
    os.makedirs(objdir, exist_ok=True)
    cflags = [f for f in FLAGS if f != "-shared"]

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *cflags, *(extra or []), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
