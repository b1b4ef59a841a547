"""Build the CPU oracle shared library with gcc (plain C, no fast-math, no FP
contraction, single thread).  Test infrastructure only."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
LIB_SAN = os.path.join(HERE, "liboracle_san.so")
# Instrumented build for the CPU tests: AddressSanitizer (out-of-bounds and
# use-after-free on the flat arrays the oracle indexes by T, k, E, H and I) and
# UndefinedBehaviorSanitizer, every finding fatal.  The instrumented library
# needs the ASan runtime loaded first (LD_PRELOAD), so the tests run it in a
# child process; see tests/test_oracle_sanitized.py.
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-fno-tree-vectorize", "-Wall", "-Wextra"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = LIB_SAN if sanitize else LIB
    cmd = ["gcc", *CFLAGS, *(SAN_FLAGS if sanitize else []), SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
