"""Build the CPU oracle (test infrastructure) into oracle/libjetfp8_oracle.so with gcc.

IEEE semantics matter for bit-exact checks: no -ffast-math, no FMA contraction (the oracle calls fmaf
explicitly where the canonical sequence has a fused multiply-add), SSE2 floating point on x86-64.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "jetfp8_oracle.c")
LIB = os.path.join(HERE, "libjetfp8_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
