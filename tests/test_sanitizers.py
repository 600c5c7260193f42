"""The CPU oracle and the library's host layer under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; no kernel is launched).

* The oracle is rebuilt with gcc -fsanitize=address,undefined (halting on
  the first report) and the pin and golden suites run against it in a child
  process.
* A copy with a planted heap overflow must be stopped by ASan, so a clean run
  means something.
* The host code of the C-ABI library (argument checks, workspace carving,
  launch planning, the no-allocation scratch) is rebuilt with host-only
  sanitizers, linked with the regular kernel objects, and every entry point
  is driven through its argument checks and size queries over a grid of
  valid and invalid shapes.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "tsv_oracle.c")
CSRC = os.path.join(ROOT, "query_aware_sparse_bbox_amd", "csrc")
OBJ = os.path.join(ROOT, "query_aware_sparse_bbox_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG_ASAN = "/opt/rocm/lib/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"


def gcc_runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build_oracle(out, source=None):
    src = ORACLE_SRC
    if source is not None:
        src = out + ".c"
        with open(src, "w") as f:
            f.write(source)
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-I", os.path.dirname(ORACLE_SRC), "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-o", out,
                    src, "-lm"], check=True)
    return out


def oracle_env(lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = gcc_runtime("libasan.so") + ":" + gcc_runtime("libubsan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["TSV_ORACLE_LIB"] = lib
    return env


def test_oracle_pins_and_golden_cases_under_asan_ubsan(tmp_path):
    lib = build_oracle(str(tmp_path / "libtsv_oracle_san.so"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_golden.py")],
                       cwd=ROOT, env=oracle_env(lib), capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert " passed" in out


def test_planted_heap_overflow_is_caught(tmp_path):
    """The same harness stops a copy of the oracle that writes one element past
    an allocation of the attention accumulator."""
    src = open(ORACLE_SRC).read()
    old = "      for (int d = 0; d < D; ++d) o[d] = (float)(acc[d] / l);"
    assert old in src
    bad = src.replace(old, "      acc[D] = 0.0; /* planted: one past the end */\n" + old)
    lib = build_oracle(str(tmp_path / "libtsv_oracle_bad.so"), bad)
    code = textwrap.dedent("""
        import workloads as W, oracle as O
        wl = W.make("tiny", context=64)
        sh = wl.shape
        meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
        O.decode_step(sh, wl.q, wl.k_pool, wl.v_pool, meta, wl.block_table, wl.seq_lens,
                      wl.k_max, wl.scale)
        print("no report")
    """)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=oracle_env(lib),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


HOST_DRIVER = textwrap.dedent(r"""
    import ctypes, itertools, sys
    L = ctypes.CDLL(sys.argv[1])

    class Shape(ctypes.Structure):
        _fields_ = [(n, ctypes.c_int32) for n in
                    ("batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size",
                     "max_pages_per_seq", "num_phys_pages", "kv_dtype")]

    class Opts(ctypes.Structure):
        _fields_ = [("n_recent", ctypes.c_int32), ("group_agg", ctypes.c_int32)]

    P_, I_, F_, Z_ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    SP, OP = ctypes.POINTER(Shape), ctypes.POINTER(Opts)
    sig = {
        "tsv_version": ([], ctypes.c_int), "tsv_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "tsv_meta_bytes": ([SP], Z_), "tsv_workspace_bytes": ([SP, I_], Z_),
        "tsv_decode_step_launches": ([SP, I_, I_], ctypes.c_int),
        "tsv_meta_build": ([SP, P_, P_, P_, P_, P_], ctypes.c_int),
        "tsv_meta_append": ([SP, P_, P_, P_, P_, P_, P_, P_, P_], ctypes.c_int),
        "tsv_select_pages_ex": ([SP, P_, P_, P_, P_, I_, P_, I_, OP, P_, P_, P_, P_, Z_, P_],
                                ctypes.c_int),
        "tsv_sparse_decode": ([SP, P_, P_, P_, P_, P_, P_, P_, I_, F_, P_, P_, Z_, P_],
                              ctypes.c_int),
        "tsv_decode_step_ex": ([SP, P_, P_, P_, P_, P_, P_, P_, P_, I_, P_, I_, OP, F_, P_, P_,
                                P_, P_, P_, Z_, P_], ctypes.c_int),
        "tsv_decode_step_noalloc": ([SP, P_, P_, P_, P_, P_, P_, P_, P_, I_, P_, I_, OP, F_, P_,
                                     P_, P_, P_, P_], ctypes.c_int),
        "tsv_schedule_rows": ([SP, I_, P_, P_, I_, I_, P_, I_, P_], ctypes.c_int),
        "tsv_decode_step_scheduled": ([SP, P_, P_, P_, P_, P_, P_, P_, P_, I_, P_, I_, OP, P_, I_,
                                       F_, P_, P_, P_, P_, P_, Z_, P_], ctypes.c_int),
    }
    for name, (a, r) in sig.items():
        f = getattr(L, name); f.argtypes = a; f.restype = r
    assert L.tsv_version() >= 1
    for st in (0, -1, -2, -3, 7, -100):
        assert L.tsv_status_string(st)
    # size queries over a grid of valid and invalid shapes
    n = 0
    for dt, D, P, G, MP, B, k in itertools.product(
            (0, 1, 2, 3, 4, 5), (64, 96, 128), (8, 12, 16, 32, 64), (1, 2, 3, 4, 8, 16, 32),
            (1, 100, 4096, 5000), (1, 64, 512), (0, 1, 64, 4096)):
        s = Shape(B, 2 * G, 2, D, P, MP, MP * B, dt)
        mb = L.tsv_meta_bytes(ctypes.byref(s))
        wb = L.tsv_workspace_bytes(ctypes.byref(s), k)
        nl = L.tsv_decode_step_launches(ctypes.byref(s), k, 1)
        valid = (dt <= 4 and D in (64, 128) and P in (8, 16, 32, 64) and G in (1, 2, 4, 8, 16)
                 and MP <= 4096)
        assert (mb > 0) == valid and ((wb > 0) == (valid and k >= 1)), (dt, D, P, G, MP, B, k)
        assert (nl > 0) == (valid and k >= 1)
        n += 1
    # every entry point rejects bad arguments before any HIP call
    s = Shape(2, 8, 2, 64, 16, 10, 20, 2)
    f = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 4)
    need = L.tsv_workspace_bytes(ctypes.byref(s), 4)
    sc = ctypes.c_float(0.1)
    o_bad = Opts(-1, 0)
    o_agg = Opts(0, 5)
    checks = [
        L.tsv_meta_build(None, f, f, f, f, None),
        L.tsv_meta_build(ctypes.byref(s), f, None, f, f, None),
        L.tsv_meta_append(ctypes.byref(s), f, None, f, f, f, f, f, None),
        L.tsv_select_pages_ex(ctypes.byref(s), None, f, f, f, 4, None, 0, None, f, f, None, f,
                              need, None),
        L.tsv_select_pages_ex(ctypes.byref(s), mis, f, f, f, 4, None, 0, None, f, f, None, f,
                              need, None),
        L.tsv_select_pages_ex(ctypes.byref(s), f, f, f, f, 4, None, 0, ctypes.byref(o_bad), f,
                              f, None, f, need, None),
        L.tsv_select_pages_ex(ctypes.byref(s), f, f, f, f, 4, None, 0, ctypes.byref(o_agg), f,
                              f, None, f, need, None),
        L.tsv_select_pages_ex(ctypes.byref(s), f, f, f, f, 4, None, 0, None, f, f, None, f,
                              need - 1, None),
        L.tsv_sparse_decode(ctypes.byref(s), f, f, f, f, f, f, f, 0, sc, f, f, need, None),
        L.tsv_sparse_decode(ctypes.byref(s), f, f, f, f, f, f, f, 4, sc, f,
                            ctypes.c_void_p((1 << 20) + 64), need, None),
        L.tsv_decode_step_ex(ctypes.byref(s), f, f, None, f, f, f, f, f, 4, None, 0, None, sc,
                             f, f, None, f, f, need, None),
        L.tsv_decode_step_ex(ctypes.byref(s), f, None, None, f, f, f, f, f, 4, None, 5, None,
                             sc, f, f, None, f, f, need, None),
        L.tsv_decode_step_noalloc(ctypes.byref(s), None, None, None, f, f, f, f, f, 4, None, 0,
                                  None, sc, f, f, None, f, None),
    ]
    assert all(c == -1 for c in checks), checks
    big = Shape(512, 8, 8, 64, 16, 4096, 1 << 20, 2)
    assert L.tsv_decode_step_noalloc(ctypes.byref(big), f, None, None, f, f, f, f, f, 64, None,
                                     0, None, sc, f, f, None, f, None) == -2
    bad_shapes = [Shape(2, 8, 2, 96, 16, 10, 20, 2), Shape(2, 6, 4, 64, 16, 10, 20, 2),
                  Shape(0, 8, 2, 64, 16, 10, 20, 2), Shape(2, 8, 2, 64, 16, 10, 20, 9)]
    for b in bad_shapes:
        assert L.tsv_decode_step_ex(ctypes.byref(b), f, None, None, f, f, f, f, f, 4, None, 0,
                                    None, sc, f, f, None, f, f, need, None) in (-1, -2)
    # the row schedule (host code only) over random lengths, budgets and CU
    # geometries: every row exactly once in a buffer of exactly its length
    import random
    rnd = random.Random(5)
    for it in range(300):
        B, Hkv = rnd.randint(1, 70), rnd.choice((1, 2, 8))
        s2 = Shape(B, Hkv * 4, Hkv, 128, 16, 64, 64 * B, rnd.randint(0, 4))
        lens = (ctypes.c_int32 * B)(*[rnd.randint(-5, 64 * 16 + 9) for _ in range(B)])
        kps = (ctypes.c_int32 * B)(*[rnd.randint(-2, 70) for _ in range(B)])
        k, cus, per = rnd.randint(1, 64), rnd.choice((1, 7, 64, 256)), rnd.randint(1, 4)
        kp = kps if it % 2 else None
        n2 = ctypes.c_int32(0)
        assert L.tsv_schedule_rows(ctypes.byref(s2), k, lens, kp, cus, per, None, 0,
                                   ctypes.byref(n2)) == 0
        buf = (ctypes.c_int32 * n2.value)()
        assert L.tsv_schedule_rows(ctypes.byref(s2), k, lens, kp, cus, per, buf, n2.value,
                                   ctypes.byref(n2)) == 0
        got = sorted(x for x in buf if x >= 0)
        assert got == list(range(B * Hkv)), it
    # the scheduled step's own checks, before any HIP call
    assert L.tsv_decode_step_scheduled(ctypes.byref(s), f, None, None, f, f, f, f, f, 4, None,
                                       0, None, ctypes.c_void_p((1 << 20) + 2), 4, sc, f, f,
                                       None, f, f, need, None) == -1
    assert L.tsv_decode_step_scheduled(ctypes.byref(s), f, None, None, f, f, f, f, f, 4, None,
                                       0, None, f, 3, sc, f, f, None, f, f, need, None) == -1
    print(f"host layer ok: {n} shapes queried")
""")


def test_host_layer_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC) or not os.path.exists(CLANG_ASAN):
        pytest.skip("hipcc or its AddressSanitizer runtime is not installed")
    kernels = sorted(os.path.join(OBJ, f) for f in os.listdir(OBJ) if f.startswith("kernels_")) \
        if os.path.isdir(OBJ) else []
    if len(kernels) != 10:
        pytest.skip("the library's kernel objects are not built (run the package build)")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
           "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), *san]
    objs = []
    for src in ("tsv_api.hip", "tsv_host.hip", "tsv_scratch.hip"):
        o = str(tmp_path / (src + ".o"))
        subprocess.run([HIPCC, *flags, "-c", "-o", o, os.path.join(CSRC, src)], check=True,
                       capture_output=True)
        objs.append(o)
    lib = str(tmp_path / "libtsv_host_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-o", lib, *objs,
                    *kernels], check=True, capture_output=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = CLANG_ASAN
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", HOST_DRIVER, lib], env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert "host layer ok" in r.stdout
