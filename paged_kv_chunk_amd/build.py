"""Build libpkc.so in-tree with hipcc for gfx950.

Usage: python -m paged_kv_chunk_amd.build  (or __graft_entry__.build()). Always recompiles.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkc.so")
ARCH = os.environ.get("PKC_OFFLOAD_ARCH", "gfx950")


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def command(out=LIB, extra=()):
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    return [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            # keep the compiler from forming packed fp32 VALU ops (device pass only; the host
            # pass warns that it does not know the feature)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in VGPRs: the online-softmax rescale of the output tiles is then a
            # plain multiply, with no copies between the accumulation and arithmetic registers
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wno-unused-command-line-argument",
            f"-I{INCLUDE}", f"-I{CSRC}", *extra, *sources, "-o", out]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = command(out=tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libpkc.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
