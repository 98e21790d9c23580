"""Build the CPU oracle (test infrastructure) into ``oracle/liboracle.so``.

Plain gcc, one translation unit, ``-O2 -ffp-contract=off`` so that the C
compiler fuses no multiply-add the source does not write as ``fmaf``.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "signmuon_oracle.c")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-fPIC", "-shared", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
