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


LIB_SAN = os.path.join(_HERE, "libattn_san.so")
# host code only (validation, planning, the C ABI): the device code is built
# as usual; each -fsanitize= goes to the host pass alone
SANITIZE_HOST = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
                 "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libsan"]


def build(verbose=False, extra=(), sanitize=False):
    """sanitize: build libattn_san.so, whose host code carries AddressSanitizer
    and UndefinedBehaviorSanitizer (see tests/sanitize.py)."""
    out = LIB_SAN if sanitize else LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = hipcc_cmd(tmp, list(extra) + (SANITIZE_HOST if sanitize else []))
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if msgs and (verbose or r.returncode != 0):
        print("\n".join(msgs), file=sys.stderr)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d)" % r.returncode)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
