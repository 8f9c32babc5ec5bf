"""Build the HIP library ``libreformer_lsh.so`` for gfx950 in-tree.

Usage: ``python -m efficient_long_sequence_lsh_amd.build`` (or ``build()``).
Every call recompiles; nothing is cached outside the package directory.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libreformer_lsh.so")
ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    out_tmp = LIB + ".tmp"
    cmd = [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # packed float32 ops stay off: ordinary float code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results in architectural VGPRs: the hash epilogue reads its 16
        # projections per lane without a v_accvgpr_read each
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
        "-o", out_tmp,
    ] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libreformer_lsh.so")
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
