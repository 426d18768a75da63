"""Build the CPU oracle library (test infrastructure; see kvq_oracle.c).

Plain gcc, -O2 with floating-point contraction off and no fast-math, so that every
binary32 step of the quantizer is one correctly rounded IEEE operation.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    """sanitize: the same library under AddressSanitizer and UndefinedBehaviorSanitizer
    (any finding aborts), written to `out`; load it with the sanitizer runtime preloaded
    (LD_PRELOAD=$(gcc -print-file-name=libasan.so)) and KVQ_ORACLE_LIB_PATH pointing at it."""
    dst = out or LIB
    san = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"] if sanitize else []
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", "-Wall", "-Wextra", *san, "-o", dst + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(dst + ".tmp", dst)
    return dst


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
