"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library must load, export every function include/tsv.h declares, report
sizes, and reject bad arguments before making any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsv.h")
TEST_HEADER = os.path.join(ROOT, "include", "tsv_testing.h")


@pytest.fixture(scope="module")
def tsv():
    import importlib.util
    path = os.path.join(ROOT, "query_aware_sparse_bbox_amd", "build.py")
    spec = importlib.util.spec_from_file_location("tsv_build", path)
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    if not os.path.exists(b.LIB):
        b.build()
    import query_aware_sparse_bbox_amd as m
    return m


def declared_functions(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(tsv_\w+)\s*\(", text, re.M)))


def exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    return set(re.findall(r" T (tsv_\w+)$", out, re.M))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("tsv_meta_append", "tsv_select_pages", "tsv_sparse_decode", "tsv_decode_step",
              "tsv_meta_build", "tsv_workspace_bytes", "tsv_meta_bytes", "tsv_status_string",
              "tsv_version", "tsv_select_pages_ex", "tsv_decode_step_ex",
              "tsv_schedule_rows", "tsv_decode_step_scheduled"):
        assert n in names


def test_library_exports_every_declared_symbol(tsv):
    ex = exported(tsv.LIB_PATH)
    for n in declared_functions():
        assert n in ex, n
        assert getattr(tsv._lib, n)
    assert set(tsv.EXPORTS) == set(declared_functions())
    # the library proper keeps no state: the testing hook is not in it
    assert not ex & set(declared_functions(TEST_HEADER))


def test_testing_library_exports_both_headers(tsv):
    ex = exported(tsv.TESTHOOKS_PATH)
    for n in declared_functions() + declared_functions(TEST_HEADER):
        assert n in ex, n
    assert set(tsv.TEST_EXPORTS) == set(declared_functions(TEST_HEADER))


@pytest.mark.parametrize("which", ["LIB_PATH", "TESTHOOKS_PATH"])
def test_library_is_built_for_gfx950(tsv, which):
    """The embedded device code targets gfx950 and nothing else."""
    data = open(getattr(tsv, which), "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-+(gfx\w+)", data))
    assert targets == {b"gfx950"}


def test_version_and_status_strings(tsv):
    assert tsv.tsv_version() == 2
    assert tsv.status_string(0) == "ok"
    assert "invalid" in tsv.status_string(-1)
    assert "unsupported" in tsv.status_string(-2)


def shape(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                max_pages_per_seq=10, num_phys_pages=20, kv_dtype=2)
    base.update(kw)
    from query_aware_sparse_bbox_amd import Shape
    return Shape(**base)


def test_sizes(tsv):
    s = shape()
    assert tsv.tsv_meta_bytes(s) == 20 * 2 * 2 * 64 * 2
    assert tsv.tsv_meta_bytes(shape(kv_dtype=0)) == 20 * 2 * 2 * 64 * 4
    assert tsv.tsv_meta_bytes(shape(kv_dtype=3)) == 20 * 2 * 2 * 64 * 1  # fp8 E4M3
    assert tsv.tsv_meta_bytes(shape(kv_dtype=4)) == 20 * 2 * 2 * 64 * 1  # fp8 E5M2
    assert tsv.tsv_meta_bytes(shape(kv_dtype=5)) == 0
    ws = tsv.tsv_workspace_bytes(s, 8)
    assert ws > 0 and ws % 256 == 0
    assert tsv.tsv_workspace_bytes(s, 16) >= ws
    assert tsv.tsv_workspace_bytes(s, 0) == 0
    assert tsv.tsv_meta_bytes(shape(head_dim=96)) == 0
    assert tsv.tsv_meta_bytes(shape(num_q_heads=7)) == 0


def test_workspace_zeroed_prefix(tsv):
    """The counters and key slots of split rows sit in a fixed
    zero-initialised prefix of the workspace (128 rows: a 128-byte line of
    counters each, then 4096 four-byte page slots each); every workspace is
    at least that large, whatever the shape."""
    text = open(HEADER).read()
    zero = int(re.search(r"#define TSV_WORKSPACE_ZERO_BYTES (\d+)", text).group(1))
    assert zero == 128 * 128 + 128 * 4096 * 4
    for s in (shape(), shape(batch=1, max_pages_per_seq=1), shape(batch=128, head_dim=128)):
        assert tsv.tsv_workspace_bytes(s, 1) > zero


def test_exchange_polls_hook_round_trip(tsv):
    """The testing library's hook only stores a number on the host (no HIP
    call); the library proper has no such state."""
    t = tsv.testing_library()
    cur = t.tsv_debug_exchange_polls(-1)
    assert cur == 16384
    assert t.tsv_debug_exchange_polls(0) == cur
    assert t.tsv_debug_exchange_polls(-1) == 0
    assert t.tsv_debug_exchange_polls(cur) == 0
    assert t.tsv_debug_exchange_polls(-1) == cur
    assert not hasattr(tsv._lib, "tsv_debug_exchange_polls")


def test_group_sizes_accepted(tsv):
    """Groups of 1, 2, 4, 8 and 16 query heads per KV head are accepted."""
    for g in (1, 2, 4, 8, 16):
        s = shape(num_q_heads=2 * g, num_kv_heads=2)
        assert tsv.tsv_workspace_bytes(s, 8) > 0, g
        assert tsv.tsv_decode_step_launches(s, 8, True) >= 1, g


def test_decode_step_launch_plan(tsv):
    # short block-table rows: the whole step of a row runs in workgroups of
    # its own, one launch (rows that leave the chip idle are spread over
    # several workgroups that merge their shares in the same kernel)
    assert tsv.tsv_decode_step_launches(shape(), 64, True) == 1
    assert tsv.tsv_decode_step_launches(shape(), 64, False) == 1
    assert tsv.tsv_decode_step_launches(shape(), 8, True) == 1
    assert tsv.tsv_decode_step_launches(shape(batch=128), 64, True) == 1
    # 8 query heads of 128 channels need more staging than one workgroup's
    # 64 KiB; 4096-entry rows with such staging too: the phases run apart
    big = shape(head_dim=128, num_q_heads=16, num_kv_heads=2, max_pages_per_seq=4096)
    assert tsv.tsv_decode_step_launches(big, 64, True) in (3, 4)
    assert tsv.tsv_decode_step_launches(big, 64, False) in (2, 3)
    assert tsv.tsv_decode_step_launches(shape(head_dim=96), 8, True) == 0
    assert tsv.tsv_decode_step_launches(shape(), 0, True) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), -2), (dict(head_dim=32), -2), (dict(page_size=12), -2),
    (dict(kv_dtype=7), -2), (dict(kv_dtype=-1), -2), (dict(num_q_heads=24, num_kv_heads=8), -2),  # G = 3
    (dict(num_q_heads=64, num_kv_heads=2), -2),  # G = 32
    (dict(num_q_heads=48, num_kv_heads=4), -2),  # G = 12
    (dict(num_q_heads=7), -1), (dict(batch=0), -1), (dict(num_phys_pages=0), -1),
    (dict(max_pages_per_seq=5000), -2),
])
def test_bad_shapes_rejected_before_any_hip_call(tsv, kw, status):
    s = shape(**kw)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: rejected first
    rc = tsv._lib.tsv_select_pages(ctypes.byref(s), fake, fake, fake, fake, 4, None, 0,
                                   fake, fake, None, fake, 1 << 30, None)
    assert rc == status


def test_bad_arguments_rejected_before_any_hip_call(tsv):
    s = shape()
    f = ctypes.c_void_p(1 << 20)
    big = 1 << 30
    L = tsv._lib
    # null required pointers
    assert L.tsv_select_pages(ctypes.byref(s), None, f, f, f, 4, None, 0, f, f, None, f, big, None) == -1
    assert L.tsv_meta_build(ctypes.byref(s), f, None, f, f, None) == -1
    assert L.tsv_meta_append(ctypes.byref(s), f, None, f, f, f, f, f, None) == -1
    # k_max / n_sink
    assert L.tsv_select_pages(ctypes.byref(s), f, f, f, f, 0, None, 0, f, f, None, f, big, None) == -1
    assert L.tsv_select_pages(ctypes.byref(s), f, f, f, f, 4, None, 5, f, f, None, f, big, None) == -1
    assert L.tsv_select_pages(ctypes.byref(s), f, f, f, f, 4, None, -1, f, f, None, f, big, None) == -1
    # misaligned q
    mis = ctypes.c_void_p((1 << 20) + 4)
    assert L.tsv_select_pages(ctypes.byref(s), mis, f, f, f, 4, None, 0, f, f, None, f, big, None) == -1
    # workspace too small or misaligned
    need = L.tsv_workspace_bytes(ctypes.byref(s), 4)
    assert L.tsv_select_pages(ctypes.byref(s), f, f, f, f, 4, None, 0, f, f, None, f, need - 1,
                              None) == -1
    assert L.tsv_select_pages(ctypes.byref(s), f, f, f, f, 4, None, 0, f, f, None,
                              ctypes.c_void_p((1 << 20) + 64), need, None) == -1
    assert L.tsv_sparse_decode(ctypes.byref(s), f, f, f, f, f, f, f, 4, ctypes.c_float(0.1), f,
                               f, need // 2, None) == -1
    assert L.tsv_decode_step(ctypes.byref(s), f, f, f, f, f, f, f, f, 4, None, 0,
                             ctypes.c_float(0.1), f, f, None, f, f, need - 1, None) == -1
    # k_new without v_new
    assert L.tsv_decode_step(ctypes.byref(s), f, f, None, f, f, f, f, f, 4, None, 0,
                             ctypes.c_float(0.1), f, f, None, f, f, need, None) == -1
    # null shape
    assert L.tsv_meta_build(None, f, f, f, f, None) == -1


@pytest.mark.parametrize("n_sink,n_recent,agg,status", [
    (0, -1, 0, -1),      # negative window
    (2, 3, 0, -1),       # sinks + window beyond k_max = 4
    (0, 0, 2, -1),       # unknown group aggregation
    (0, 0, -1, -1),
])
def test_bad_selection_options_rejected_before_any_hip_call(tsv, n_sink, n_recent, agg, status):
    s = shape()
    f = ctypes.c_void_p(1 << 20)
    L = tsv._lib
    need = L.tsv_workspace_bytes(ctypes.byref(s), 4)
    o = ctypes.byref(tsv.SelectOpts(n_recent, agg))
    assert L.tsv_select_pages_ex(ctypes.byref(s), f, f, f, f, 4, None, n_sink, o, f, f, None, f,
                                 need, None) == status
    assert L.tsv_decode_step_ex(ctypes.byref(s), f, None, None, f, f, f, f, f, 4, None, n_sink,
                                o, ctypes.c_float(0.1), f, f, None, f, f, need, None) == status


def test_noalloc_rejects_shapes_beyond_its_scratch_before_any_hip_call(tsv):
    """The no-allocation step checks its arguments, then that the shape's
    scratch fits the library-owned array, before any HIP call."""
    f = ctypes.c_void_p(1 << 20)
    L = tsv._lib
    big = shape(batch=512, num_q_heads=8, num_kv_heads=8, max_pages_per_seq=4096,
                num_phys_pages=1 << 20)
    assert L.tsv_workspace_bytes(ctypes.byref(big), 64) > 33554432
    assert L.tsv_decode_step_noalloc(ctypes.byref(big), f, None, None, f, f, f, f, f, 64, None,
                                     0, None, ctypes.c_float(0.1), f, f, None, f, None) == -2
    s = shape()
    # the same argument checks as the workspace entry point
    assert L.tsv_decode_step_noalloc(ctypes.byref(s), None, None, None, f, f, f, f, f, 4, None,
                                     0, None, ctypes.c_float(0.1), f, f, None, f, None) == -1
    assert L.tsv_decode_step_noalloc(ctypes.byref(s), f, f, None, f, f, f, f, f, 4, None,
                                     0, None, ctypes.c_float(0.1), f, f, None, f, None) == -1
    assert L.tsv_decode_step_noalloc(ctypes.byref(s), f, None, None, f, f, f, f, f, 0, None,
                                     0, None, ctypes.c_float(0.1), f, f, None, f, None) == -1


def test_scheduled_step_rejects_bad_orders_before_any_hip_call(tsv):
    """The scheduled step checks its row order (4-byte aligned, at least one
    entry per row, at most 2^24) after the step's own checks, before any HIP
    call; the residency query checks its outputs before querying."""
    f = ctypes.c_void_p(1 << 20)
    L = tsv._lib
    s = shape()  # 2 sequences x 2 KV heads
    need = L.tsv_workspace_bytes(ctypes.byref(s), 4)
    sc = ctypes.c_float(0.1)

    def step(order, n, q=f, ws_bytes=need):
        return L.tsv_decode_step_scheduled(ctypes.byref(s), q, None, None, f, f, f, f, f, 4,
                                           None, 0, None, order, n, sc, f, f, None, f, f,
                                           ws_bytes, None)

    assert step(ctypes.c_void_p((1 << 20) + 2), 4) == -1   # misaligned
    assert step(f, 3) == -1                                  # fewer entries than rows
    assert step(f, (1 << 24) + 1) == -1                      # beyond the limit
    assert step(f, 4, q=None) == -1                          # the step's own checks
    assert step(f, 4, ws_bytes=need - 1) == -1
    assert step(None, 0, q=None) == -1
    one = ctypes.c_int32(0)
    assert L.tsv_step_residency(ctypes.byref(s), 4, None, ctypes.byref(one)) == -1
    assert L.tsv_step_residency(ctypes.byref(s), 0, ctypes.byref(one), ctypes.byref(one)) == -1
    assert L.tsv_step_residency(None, 4, ctypes.byref(one), ctypes.byref(one)) == -1


def test_one_hip_runtime_whatever_the_import_order():
    """Imported before torch, the package still binds the library to torch's
    HIP runtime: a process must not hold two HIP runtimes (the library's
    launches would then not see torch's memory)."""
    code = ("import query_aware_sparse_bbox_amd, torch\n"
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run(["python3", "-c", code], capture_output=True, text=True, check=True,
                         cwd=ROOT, timeout=300).stdout.strip().splitlines()[-1]
    libs = eval(out)
    assert len(libs) == 1, libs
