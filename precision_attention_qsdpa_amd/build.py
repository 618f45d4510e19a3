"""Builds ``libqsdpa.so`` in-tree with hipcc for gfx950.

Usage: ``python -m precision_attention_qsdpa_amd.build`` (or ``build()``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqsdpa.so")
SOURCES = ["qsdpa_api.cpp", "qsdpa_quant.hip", "qsdpa_attn.hip", "qsdpa_vc.hip", "qsdpa_noalloc.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division and square root; no contraction unless written out
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-ffp-contract=off",
    # keep the next step's score MFMAs in the block where they are written, so
    # they interleave with the softmax instead of sinking past its branch
    "-mllvm", "-disable-machine-sink",
    # MFMA results and accumulators in VGPRs: the softmax and the rescale work
    # on them with VALU instructions, which cannot read AGPRs without copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libqsdpa.so")
    return path


# The race-detection build: the same sources with QSDPA_RING_STRESS, which
# makes every wave sleep pseudo-random times where the attention kernels'
# tile ring hands stages between waves (its output must be bit-identical).
STRESS_LIB = os.path.join(PKG, "libqsdpa_stress.so")


def _compile(out: str, extra: list, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc()] + FLAGS + extra + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source into libqsdpa.so, and the race-detection build
    libqsdpa_stress.so (always recompiles both)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(2) as ex:
        jobs = [ex.submit(_compile, LIB, [], verbose),
                ex.submit(_compile, STRESS_LIB, ["-DQSDPA_RING_STRESS=1"], verbose)]
        for j in jobs:
            j.result()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
