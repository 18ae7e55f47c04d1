"""Run the CPU test suite against host-sanitized builds.

    python tests/sanitize.py [extra pytest args]

Builds liboracle_san.so (the oracle with clang's AddressSanitizer and
UndefinedBehaviorSanitizer) and libattn_san.so (the library with the same
sanitizers on its host code: argument validation, planning, the C ABI; the
device code is built as usual), then runs ``pytest -m "not gpu"`` in a child
process that preloads clang's sanitizer runtime and loads both builds.  Leak
detection is off (the Python interpreter keeps its allocations to the end);
any other report aborts the run.  Not collected by pytest (no test_ prefix).
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main(args):
    from causal_gqa_prefill_flash_amd import build as hipbuild
    from oracle import build as obuild
    oracle_lib = obuild.build(sanitize=True)
    attn_lib = hipbuild.build(sanitize=True)
    rt = sorted(glob.glob(os.path.join(obuild.LLVM, "lib", "clang", "*", "lib", "linux",
                                       "libclang_rt.asan-x86_64.so")))
    if not rt:
        raise SystemExit("clang's AddressSanitizer runtime was not found under " + obuild.LLVM)
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt[-1], ATTN_LIB_PATH=attn_lib, ORACLE_LIB_PATH=oracle_lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
           "-p", "no:cacheprovider"] + list(args)
    print("sanitized run:", attn_lib, oracle_lib, rt[-1], flush=True)
    try:
        return subprocess.call(cmd, env=env, cwd=ROOT)
    finally:
        # the sanitized builds are for this run only
        for p in (attn_lib, oracle_lib):
            if os.path.exists(p):
                os.remove(p)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
