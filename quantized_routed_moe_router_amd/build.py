"""Build libds4moe.so in-tree with hipcc for gfx950.

    python quantized_routed_moe_router_amd/build.py   (does not import the package)
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libds4moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 instructions are kept out of the generated code on purpose.
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # keep MFMA accumulators in VGPRs: the scale corrections read them every super-block
         "-mllvm", "-amdgpu-mfma-vgpr-form=true",
         # no sinking of common code into a shared successor.  The prefill GEMM has one inlined
         # multiply instance per live n-tile count; each ends in the same stores, which the sinking
         # merges into one store fed by a phi of the instances' 128-bit results.  This compiler's
         # register coalescer then gave lanes 1-3 of one instance's loop-carried accumulator the
         # registers that its loop uses as temporaries (wrong values in the last n-tile of the second
         # row tile of the down projection; turning off global copy coalescing removed them too)
         "-mllvm", "-simplifycfg-sink-common=false",
         "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
