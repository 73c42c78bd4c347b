"""Compile libpbsa.so for gfx950 in-tree with hipcc (no GPU needed: hipcc cross-compiles)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpbsa.so")
SOURCES = ["api.hip", "estimate.hip", "prefix_rank.hip", "sample_attn.hip", "attention.hip"]
# MFMA accumulators stay in VGPRs: the fp64 kernels otherwise move every accumulator between the
# AGPR and VGPR files around each MFMA.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# Per-source extra flags.  The attention and estimation sources: no NaN is produced or tested there
# (masked scores and logits are -inf, and every -inf path is selected away before it could meet an
# opposite infinity), so max and compare need no NaN quieting; api.hip validates arguments with
# comparisons that must keep their NaN meaning and gets no such flag.
SOURCE_FLAGS = {
    "api.hip": VGPR_FORM,
    "estimate.hip": VGPR_FORM + ["-fno-honor-nans"],
    "prefix_rank.hip": VGPR_FORM,
    "sample_attn.hip": VGPR_FORM,
    "attention.hip": VGPR_FORM + ["-fno-honor-nans"],
}

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU forms are kept out of generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build_library(verbose: bool = False) -> str:
    """Build libpbsa.so next to this file (always recompiles) and return its path."""
    import tempfile
    with tempfile.TemporaryDirectory(prefix="pbsa_build_") as tmpdir:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
            _run([hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
                  os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp = LIB + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
