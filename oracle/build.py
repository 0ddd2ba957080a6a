"""Builds the oracle's C part (test infrastructure only).

Compiles ``arx_oracle.c`` into ``liboracle.so`` next to it with gcc: no
fast-math and no floating-point contraction, so every binary32 add in the
reduction is one IEEE round-to-nearest-even add.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "arx_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-fPIC", "-shared", "-std=c11",
        "-fno-fast-math", "-ffp-contract=off", "-pthread",
        SRC, "-o", LIB + ".tmp",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
