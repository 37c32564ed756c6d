"""Build the gfx950 library libgr.so in-tree with hipcc.

    python -m trie_constrained_beam_step_amd.build [-v]

Compiles csrc/*.hip for --offload-arch=gfx950 into
trie_constrained_beam_step_amd/libgr.so (the C ABI of include/gr.h).
--sanitize builds libgr_san.so instead: the host code under AddressSanitizer
and UndefinedBehaviorSanitizer (tests/run_sanitized.py uses it).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgr.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("GR_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # no packed fp32 instructions are generated (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every rounding is the source's: a product is never fused into the sum
    # that follows it (the intrinsics __fmul_rn / __fadd_rn are plain * and +
    # here, and the scores' fp32 steps must round as written); the kernels'
    # fused multiply-adds are explicit fmaf calls
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


# host code only, under AddressSanitizer and UndefinedBehaviorSanitizer
# (device code is built as usual); loaded with clang's ASan runtime preloaded
LIB_SAN = os.path.join(HERE, "libgr_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = LIB_SAN if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    msg = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
