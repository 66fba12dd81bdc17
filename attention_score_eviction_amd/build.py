"""Build libkvsel.so in-tree with hipcc for gfx950.

Usage: python -m attention_score_eviction_amd.build   (or build() from Python)
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkvsel.so")

ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if os.path.exists(cand):
        return cand
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found: the kvsel library needs the ROCm toolchain")
    return found


def command(out: str = LIB) -> list[str]:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from forming packed-fp32 instructions by itself
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core results straight into VGPRs: the score passes read every
        # logit with VALU instructions, so accumulator-register copies would
        # cost one extra instruction per logit
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
        *srcs, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source of the package into libkvsel.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
