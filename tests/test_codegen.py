"""The hot kernel instantiations compile without register spills.

The streaming row kernel runs at its register limit (six 256-thread
workgroups per CU); a spill puts scratch traffic into the stream loop of
every step.  This compiles the device code for gfx950 (no GPU needed) and
reads each kernel's private-segment size from the code object's metadata.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "trie_constrained_beam_step_amd", "csrc")
ROCM = "/opt/rocm"

# (source, kernel name pattern): the workloads' hot instantiations
HOT = [
    ("row_kernel.hip", r"row_kernelItLi256ELi0E"),   # bf16 rows, 256 threads, streamed (the LLM-vocabulary rows)
    ("row_kernel.hip", r"row_kernelIfLi64ELi0E"),    # fp32 rows <= 4,096 tokens (SID-only, deep trie, tiny)
    ("row_kernel.hip", r"row_kernelIfLi256ELi0E"),   # fp32 long trie rows
    ("row_kernel.hip", r"row_kernelIfLi256ELi4E"),   # fp32 unconstrained rows (the EOS workload's dense rows)
    ("fused_kernel.hip", r"fused_step_kernelIfE"),
    ("fused_kernel.hip", r"fused_step_kernelItE"),
    ("fused_kernel.hip", r"fused_rows_kernelIfE"),
    ("fused_kernel.hip", r"fused_rows_kernelItE"),
    ("fused_kernel.hip", r"merge_kernel"),
    ("fused_kernel.hip", r"fused_search_kernelIfE"),   # one-launch searches of one-workgroup steps
    ("fused_kernel.hip", r"fused_search_kernelItE"),
    ("select_kernel.hip", r"select_kernelItE"),
    ("select_kernel.hip", r"select_kernelIfE"),
]


def _private_sizes(src, tmp):
    obj = os.path.join(tmp, "k.o")
    dev = os.path.join(tmp, "k.gfx950.o")
    subprocess.run([f"{ROCM}/bin/hipcc", "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-c",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, src), "-o", obj],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    subprocess.run([f"{ROCM}/llvm/bin/clang-offload-bundler", "--unbundle", "--type=o", f"--input={obj}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={dev}"], check=True)
    notes = subprocess.run([f"{ROCM}/llvm/bin/llvm-readelf", "--notes", dev], check=True,
                           stdout=subprocess.PIPE, text=True).stdout
    out, name = {}, None
    for line in notes.splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            name = m.group(1)
        m = re.match(r"\s+\.private_segment_fixed_size:\s+(\d+)", line)
        if m and name:
            out[name] = int(m.group(1))
    return out


@pytest.mark.skipif(not os.path.exists(f"{ROCM}/bin/hipcc"), reason="no hipcc")
def test_hot_kernels_have_no_scratch(tmp_path):
    by_src = {}
    for src, _ in HOT:
        if src not in by_src:
            by_src[src] = _private_sizes(src, str(tmp_path))
    for src, pat in HOT:
        hits = {k: v for k, v in by_src[src].items() if re.search(pat, k)}
        assert hits, (src, pat, sorted(by_src[src]))
        for k, v in hits.items():
            assert v == 0, f"{k} uses {v} bytes of scratch (register spills)"
