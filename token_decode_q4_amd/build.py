"""Build the HIP library (gfx950) in-tree: token_decode_q4_amd/libqd.so."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqd.so")
SOURCES = [os.path.join(HERE, "csrc", "qd_api.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions: the compiler would otherwise form them from plain float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results straight into VGPRs: the batched products read each
    # block's result once, and the AGPR form adds a copy per value
    "-mllvm", "--amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
