"""Runs the CPU test suite (pytest -m "not gpu") against AddressSanitizer +
UBSan builds of the host code: the oracle (liboracle_san.so), the host input
generator (libmoe_synth_san.so) and the host side of the HIP library
(libmoe_mxfp4_san.so: argument validation and launch set-up; its device code
is unchanged).  All three use clang's sanitizer runtime, which is preloaded
into the test process.

    python tests/run_sanitized.py [extra pytest args]
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main() -> int:
    import oracle
    from mxfp4_routed_expert_02_amd import build, synth

    oracle.build(verbose=True, sanitize=True)
    synth.build(verbose=True, sanitize=True)
    build.build_library(verbose=True, sanitize=True)
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        print("clang's ASan runtime was not found under /opt/rocm/llvm", file=sys.stderr)
        return 2
    env = dict(os.environ, MOE_SANITIZE="1", LD_PRELOAD=rt[-1],
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", "-p",
           "no:cacheprovider"] + sys.argv[1:]
    print(" ".join(cmd), flush=True)
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main())
