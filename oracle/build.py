"""Build the CPU oracle shared library with gcc (test infrastructure only)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "_build", "libqd_oracle.so")


def compile_source(src: str, out: str) -> str:
    """Compile one C source of the oracle into a shared library at ``out``."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = ["gcc", "-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-std=c11",
           "-Wall", "-Wextra", "-I", HERE, "-shared", "-fPIC", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB):
        return LIB
    return compile_source(os.path.join(HERE, "qd_oracle.c"), LIB)


if __name__ == "__main__":
    print(build())
