"""Build libh3attn.so in-tree with hipcc for gfx950.

Usage: python -m packed_full_attention_amd.build [--verbose]

Device flags, stated on purpose:
  -O3 --offload-arch=gfx950    CDNA4 only; no other GPU target is built.
  -ffp-contract=off            no compiler-chosen FMA contraction; the kernels
                               write every fused multiply-add they use.
  -fno-fast-math (default)     accurate sqrt, division, sin/cos/pow.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                               no packed-fp32 (v_pk_*_f32) instructions.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libh3attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

DEVICE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-instruction accumulators in VGPRs even in kernels that use more
    # than 256 registers (the one-wave-per-SIMD dK/dV kernel): its scores are
    # read by vector instructions, and the AGPR half then holds the operands
    # that only the matrix cores read.  The other kernels compile to the same code.
    "-mllvm", "--amdgpu-mfma-vgpr-form",
]
HOST_FLAGS = ["-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libh3attn)")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, out_path: str = LIB_PATH, extra_flags: list[str] | None = None) -> str:
    """Compile every HIP/C++ source under csrc/ into one shared library."""
    cmd = [hipcc(), *DEVICE_FLAGS, *HOST_FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC,
           *(extra_flags or []), "-o", out_path + ".tmp", *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so; drop that noise.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and "ignoring feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out_path + ".tmp", out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
