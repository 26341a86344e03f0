"""Compile the gfx950 HIP library in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", name) for name in ("attn_fwd.hip", "attn_fwd_f8.hip", "attn_bwd.hip", "attn_decode.hip")]
LIBRARY = os.path.join(PKG, "libattn_gfx950.so")
CALIBRATE_SOURCE = os.path.join(PKG, "csrc", "calibrate_gfx950.hip")
CALIBRATE = os.path.join(PKG, "calibrate_gfx950")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs: the softmax rescales them with
    # VALU ops, which cannot read AGPRs without a copy each way
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]
HIPCC_FLAGS = COMMON_FLAGS + ["-fPIC", "-shared"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    """Compile the library ``libattn_gfx950.so`` and the ``calibrate_gfx950``
    tool (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIBRARY + ".tmp"
    _run([hipcc, *HIPCC_FLAGS, "-o", tmp, *SOURCES], verbose)
    os.replace(tmp, LIBRARY)
    tmp = CALIBRATE + ".tmp"
    _run([hipcc, *COMMON_FLAGS, "-o", tmp, CALIBRATE_SOURCE], verbose)
    os.replace(tmp, CALIBRATE)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
