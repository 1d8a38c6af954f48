"""Compile the HIP sources of the engine into the in-tree shared library libjolt.so (gfx950)."""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libjolt.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code.  hipcc hands
    # -Xclang options to the host pass as well, and the driver refuses to scope -Xclang to
    # the device pass with -Xarch_device; the x86 pass ignores the feature with a warning
    # (filtered below), the gfx950 pass applies it.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]

# the host pass's notice about the device-only feature above
_HARMLESS = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if l.strip() and _HARMLESS not in l)
    if out:
        sys.stderr.write(out + "\n")
    if r.returncode != 0:
        raise RuntimeError("hipcc failed building libjolt.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
