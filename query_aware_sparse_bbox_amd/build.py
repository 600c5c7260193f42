"""Build libtsv.so (the C-ABI library and its gfx950 kernels) in place.

hipcc cross-compiles for gfx950 without a GPU.  Flags:
  -ffp-contract=off   no implicit multiply-add fusion: page scores must match
                      the fixed rounding sequence bit for bit (attention code
                      writes its fused multiply-adds explicitly);
  -packed-fp32-ops    disabled: no packed fp32 VALU instructions are emitted.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libtsv.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("tsv_api.hip", "tsv_kernels.hip")]
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.exists(c) or c == "hipcc"):
            return c
    raise RuntimeError("hipcc not found")


def build(extra_flags=(), verbose=False):
    out = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           "-I", os.path.join(ROOT, "include"), *extra_flags, "-o", out, *SOURCES]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
