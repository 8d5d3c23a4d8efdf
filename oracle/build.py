"""Build the fp64 CPU oracle library (test infrastructure).

gcc -O2 -fopenmp, no fast-math: the oracle must evaluate its sums in the
written order.  Output: oracle/libssd_oracle.so next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "ssd_recurrence.c"), os.path.join(HERE, "ssd_recurrence_bwd.c")]
LIB = os.path.join(HERE, "libssd_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", *SRCS, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
