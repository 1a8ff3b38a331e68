"""Compile the oracle's C part with gcc (host code only, no HIP).

Test infrastructure: the library built here is loaded only by the tests, the
package smoke check and the benchmark's CPU-baseline leg.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_attn.so")
SRC = os.path.join(HERE, "attn_oracle.c")


def build(verbose: bool = False) -> str:
    # -ffp-contract=off keeps every multiply and add separately rounded, so the
    # double-precision sums are the plain left-to-right ones written in the source.
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
