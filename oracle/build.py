"""Build the CPU oracle (liboracle.so) with gcc.

Test infrastructure: the oracle is compiled by the package build step so that the
checker exists, but only the tests, the smoke check and the benchmark's cpu_baseline
leg load it.  Flags: no fast-math, no implicit FMA contraction (-ffp-contract=off);
-mfma only lets the explicit fmaf() calls compile to the hardware instruction.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    cmd = ["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-o", LIB + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
