"""Build liboracle.so from oracle.c with the host C compiler (test infrastructure).

IEEE double arithmetic throughout: no -ffast-math and no FMA contraction, so
the oracle's rounding is that of the plain C expressions it contains.
"""
import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))


LLVM = "/opt/rocm/llvm"


def build(verbose=False, sanitize=False):
    """sanitize: build liboracle_san.so instead, with clang's AddressSanitizer
    and UndefinedBehaviorSanitizer (the same runtime as the library's host
    sanitizer build, so both load into one process; see tests/sanitize.py)."""
    src = os.path.join(_HERE, "oracle.c")
    out = os.path.join(_HERE, "liboracle_san.so" if sanitize else "liboracle.so")
    tmp = out + ".tmp%d" % os.getpid()
    cc = os.path.join(LLVM, "bin", "clang") if sanitize else "gcc"
    cmd = [cc, "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-std=c11", "-Wall", "-o", tmp, src, "-lm"]
    if sanitize:
        cmd[1:1] = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-shared-libsan",
                    "-L" + os.path.join(LLVM, "lib"), "-Wl,-rpath," + os.path.join(LLVM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
