"""Build libtsv.so (the C-ABI library and its gfx950 kernels) in place.

hipcc cross-compiles for gfx950 without a GPU.  The kernel source is compiled
once per KV type and kernel family (phased kernels, one-launch step) into
separate objects, in parallel, then linked with the host layer into

  libtsv.so             the library proper (include/tsv.h)
  libtsv_testhooks.so   the same entry points plus the testing hooks of
                        include/tsv_testing.h; its one-launch step kernels
                        record phase stamps (-DTSV_PHASE_STAMPS)

Flags:
  -ffp-contract=off   no implicit multiply-add fusion: page scores must match
                      the fixed rounding sequence bit for bit (attention code
                      writes its fused multiply-adds explicitly);
  -packed-fp32-ops    disabled: no packed fp32 VALU instructions are emitted;
  -amdgpu-kernarg-preload-count=16
                      the first kernel arguments arrive in scalar registers
                      with the wave instead of through a load (the compiler
                      takes as many as the free user registers hold, 14 dwords
                      for the step kernel, and keeps a fallback that loads
                      them for firmware without preloading).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtsv.so")
LIB_TESTHOOKS = os.path.join(PKG, "libtsv_testhooks.so")
ARCH = "gfx950"
KV_TYPES = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3, "e5m2": 4}
PARTS = {"phased": 0, "step": 1}


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.exists(c) or c == "hipcc"):
            return c
    raise RuntimeError("hipcc not found")


def flags(extra=()):
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), *extra]


def units(extra=()):
    """(object path, compile command) of every translation unit."""
    out = []

    def cc(src, name, defs=()):
        obj = os.path.join(OBJ, name + ".o")
        out.append((obj, [hipcc(), *flags(extra), *defs, "-c", "-o", obj,
                          os.path.join(CSRC, src)]))
        return obj

    for tname, t in KV_TYPES.items():
        for pname, p in PARTS.items():
            cc("tsv_kernels.hip", f"kernels_{tname}_{pname}", [f"-DTSV_DT={t}", f"-DTSV_PART={p}"])
        # the testing library's step kernels record phase stamps
        cc("tsv_kernels.hip", f"stamped_{tname}_step",
           [f"-DTSV_DT={t}", f"-DTSV_PART={PARTS['step']}", "-DTSV_PHASE_STAMPS"])
    cc("tsv_host.hip", "host")
    cc("tsv_scratch.hip", "scratch")
    cc("tsv_api.hip", "api")
    cc("tsv_api.hip", "api_testhooks", ["-DTSV_TEST_HOOKS"])
    return out


def build(extra_flags=(), verbose=False, jobs=None):
    os.makedirs(OBJ, exist_ok=True)
    todo = units(extra_flags)
    jobs = jobs or max(1, min(len(todo), os.cpu_count() or 1, 16))

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    with ThreadPoolExecutor(max_workers=jobs) as pool:
        list(pool.map(run, [c for _, c in todo]))
    objs = {os.path.basename(o)[:-2]: o for o, _ in todo}
    kernels = [o for n, o in objs.items() if n.startswith("kernels_")]
    testing = [o for n, o in objs.items()
               if n.startswith("stamped_") or (n.startswith("kernels_") and n.endswith("_phased"))]
    for lib, api, kobjs in ((LIB, "api", kernels), (LIB_TESTHOOKS, "api_testhooks", testing)):
        tmp = lib + ".tmp"
        run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, objs[api],
             objs["host"], objs["scratch"], *kobjs])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
