"""Build the fp64 CPU oracle (test infrastructure) into oracle/libgdn2_oracle.so.

Plain gcc, -O2, no fast-math: the oracle's rounding must follow IEEE fp64.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn2_oracle.c")
SRCS = [SRC, os.path.join(HERE, "gdn2_oracle_bwd.c")]
LIB = os.path.join(HERE, "libgdn2_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           *SRCS, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
