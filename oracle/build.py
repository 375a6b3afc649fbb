"""Build the CPU oracle (test infrastructure) into oracle/libkvarn_oracle.so.

Plain gcc, IEEE double arithmetic: no -ffast-math and no FMA contraction, so
every operation in kvarn_oracle.c rounds exactly as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvarn_oracle.c")
LIB = os.path.join(HERE, "libkvarn_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
