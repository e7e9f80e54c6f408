"""Build the KIVI reference oracle (test infrastructure only) with gcc.

The oracle is compiled with floating-point contraction off and without
fast-math or -march flags, so every float operation is one IEEE binary32
operation rounded to nearest even.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kivi_oracle.c")
LIB = os.path.join(HERE, "libkivi_oracle.so")

CMD = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
       "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB, SRC, "-lm"]


def build(verbose: bool = False) -> str:
    if verbose:
        print(" ".join(CMD), flush=True)
    subprocess.run(CMD, check=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
