"""Build libattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Packed fp32 VALU instructions are disabled for the device code
(-target-feature -packed-fp32-ops); the host pass warns that it does not
know the feature, which is harmless.
"""
import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB = os.path.join(_HERE, "libattn.so")
SOURCES = [os.path.join(_HERE, "csrc", "attn.hip")]


def hipcc_cmd(out, extra=()):
    return (["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-shared", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(_ROOT, "include"), "-o", out] + list(extra) + SOURCES)


def build(verbose=False, extra=()):
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_cmd(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if msgs and (verbose or r.returncode != 0):
        print("\n".join(msgs), file=sys.stderr)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d)" % r.returncode)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
