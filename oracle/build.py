"""Build liboracle.so from oracle.c with the host C compiler (test infrastructure).

IEEE double arithmetic throughout: no -ffast-math and no FMA contraction, so
the oracle's rounding is that of the plain C expressions it contains.
"""
import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose=False):
    src = os.path.join(_HERE, "oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-std=c11", "-Wall", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
