"""Build the fp64 CPU oracle (test infrastructure) as oracle/liboracle.so.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark load
the result.  gcc with OpenMP; no target-specific flags, so the library runs on
any x86-64 host of the same image.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-Wno-unused-parameter", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
