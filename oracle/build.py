"""Compile the CPU oracle (fp8_oracle.c) into liboracle.so, in place.

Test infrastructure: the oracle is built with the product so the checks can run,
but nothing on the product path loads it."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # IEEE semantics: no fast-math, no contraction of a*b+c into fma.
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", "-fno-builtin-rint",
           os.path.join(HERE, "fp8_oracle.c"), "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
