"""Build libmoe_fp4.so (gfx950) in-tree with hipcc.

    python -m block_scaled_fp4_gather_amd.build

Packed-fp32 VALU forms are disabled for all device code
(-target-feature -packed-fp32-ops); the host pass warns that it does not
know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_fp4.so")
SOURCES = ["api.hip", "prepare.hip", "decode_path.hip", "prefill.hip", "prefill_a8.hip", "mxfp8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def command(out: str) -> list[str]:
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmoe_fp4.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
