"""Compile the fp64 oracle (plain C) into a shared library beside its source.

Test infrastructure: the oracle is the checker, not the product.  It is built
with gcc at -O2 and without fast-math so that libm's exp/expm1/log1p are used
as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssm_oracle.c")
LIB = os.path.join(HERE, "libssm_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm", "-pthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
