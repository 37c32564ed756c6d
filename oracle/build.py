"""Build the C oracle (test infrastructure) into oracle/liboracle.so with gcc.

IEEE semantics are kept: no -ffast-math, and -ffp-contract=off so that no
multiply-add is fused.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


# the same source under AddressSanitizer and UndefinedBehaviorSanitizer, built
# by the clang whose ASan runtime the sanitized GPU library's host code uses
# (one runtime per process; tests/run_sanitized.py)
LIB_SAN = os.path.join(HERE, "liboracle_san.so")
CLANG = "/opt/rocm/llvm/bin/clang"


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = LIB_SAN if sanitize else LIB
    cc = [CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-g"] if sanitize else ["gcc"]
    cmd = [*cc, "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
