"""The CPU test suite (-m "not gpu") against host-sanitized builds.

    python tests/run_sanitized.py [extra pytest args]

Builds libgr_san.so (the library's host code -- argument and trie
validation, planning, the C ABI -- under AddressSanitizer and
UndefinedBehaviorSanitizer; device code as usual) and liboracle_san.so (the C
oracle under the same sanitizers, by the same clang), then runs the CPU tests
in a child process that preloads clang's ASan runtime and loads those builds
(GR_LIBRARY, GRO_LIBRARY).  Any report aborts the run: every sanitizer stops
at its first finding.  Leak checking is off: the interpreter keeps its own
allocations until exit.
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main() -> int:
    from oracle import build as oracle_build
    from trie_constrained_beam_step_amd import build as gr_build
    lib = gr_build.build(verbose=True, sanitize=True)
    olib = oracle_build.build(verbose=True, sanitize=True)
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        print("clang's ASan runtime is not installed", file=sys.stderr)
        return 2
    env = dict(os.environ, LD_PRELOAD=rts[-1], GR_LIBRARY=lib, GRO_LIBRARY=olib, PYTHONMALLOC="malloc",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q",
           "-p", "no:cacheprovider", *sys.argv[1:]]
    print("LD_PRELOAD=" + rts[-1], " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
