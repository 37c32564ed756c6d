"""Build tests/c/abi_demo (plain C against the library's C ABI and the C
oracle; test infrastructure).

    python tests/c/build_demo.py

gcc, linked to libgr.so, liboracle.so and the HIP runtime, with run paths to
the in-tree libraries (build those first)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
OUT = os.path.join(HERE, "abi_demo")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "trie_constrained_beam_step_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", orc, "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "abi_demo.c"), "-o", OUT + ".tmp",
           "-L", pkg, "-lgr", "-L", orc, "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-lm", "-Wl,-rpath,$ORIGIN/../../trie_constrained_beam_step_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{r.stdout}")
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
