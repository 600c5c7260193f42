"""Python binding of libtsv: query-aware page selection + sparse paged decode.

Argument marshalling only.  Every function takes torch tensors that already
live on the current HIP device, passes their data pointers and a stream to the
C ABI declared in ``include/tsv.h`` and raises :class:`TsvError` on a non-zero
status.  Nothing here computes any part of the method, and there is no
fallback: importing this module fails when ``libtsv.so`` is not built.
"""
from __future__ import annotations

import ctypes
import os

# torch first: it carries its own HIP runtime, and the library must bind to
# that one (the runtime that owns the tensors' memory and streams), not load a
# second copy from the system ROCm when imported before torch
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtsv.so")
# the same kernels and entry points plus the testing hook of
# include/tsv_testing.h (tests only)
TESTHOOKS_PATH = os.path.join(_HERE, "libtsv_testhooks.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; build it with "
        "`python query_aware_sparse_bbox_amd/build.py` (hipcc, gfx950)")

TSV_F32, TSV_F16, TSV_BF16, TSV_FP8_E4M3, TSV_FP8_E5M2 = 0, 1, 2, 3, 4
TSV_OK, TSV_ERR_INVALID_ARG, TSV_ERR_UNSUPPORTED, TSV_ERR_HIP = 0, -1, -2, -3
TSV_AGG_MAX, TSV_AGG_SUM = 0, 1

# functions declared in include/tsv.h (all exported by both libraries)
EXPORTS = ("tsv_version", "tsv_status_string", "tsv_meta_bytes", "tsv_workspace_bytes",
           "tsv_decode_step_launches", "tsv_meta_build", "tsv_meta_append",
           "tsv_select_pages", "tsv_sparse_decode", "tsv_decode_step",
           "tsv_select_pages_ex", "tsv_decode_step_ex", "tsv_decode_step_noalloc",
           "tsv_schedule_rows", "tsv_step_residency", "tsv_decode_step_scheduled")
# declared in include/tsv_testing.h, exported by the testing library only
TEST_EXPORTS = ("tsv_debug_exchange_polls", "tsv_debug_phase_stamps")


class TsvError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


class Shape(ctypes.Structure):
    """tsv_shape."""
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size",
                 "max_pages_per_seq", "num_phys_pages", "kv_dtype")]

    @classmethod
    def of(cls, s) -> "Shape":
        """From any object with the eight tsv_shape fields."""
        return cls(*(int(getattr(s, n)) for n, _ in cls._fields_))


class SelectOpts(ctypes.Structure):
    """tsv_select_opts."""
    _fields_ = [("n_recent", ctypes.c_int32), ("group_agg", ctypes.c_int32)]


_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_SP = ctypes.POINTER(Shape)
_OP = ctypes.POINTER(SelectOpts)
_SIGS = {
    "tsv_version": ([], ctypes.c_int),
    "tsv_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "tsv_meta_bytes": ([_SP], _Z),
    "tsv_workspace_bytes": ([_SP, _I], _Z),
    "tsv_decode_step_launches": ([_SP, _I, _I], ctypes.c_int),
    "tsv_meta_build": ([_SP, _P, _P, _P, _P, _P], ctypes.c_int),
    "tsv_meta_append": ([_SP, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "tsv_select_pages": ([_SP, _P, _P, _P, _P, _I, _P, _I, _P, _P, _P, _P, _Z, _P],
                         ctypes.c_int),
    "tsv_sparse_decode": ([_SP, _P, _P, _P, _P, _P, _P, _P, _I, _F, _P, _P, _Z, _P],
                          ctypes.c_int),
    "tsv_decode_step": ([_SP, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _F, _P, _P, _P,
                         _P, _P, _Z, _P], ctypes.c_int),
    "tsv_select_pages_ex": ([_SP, _P, _P, _P, _P, _I, _P, _I, _OP, _P, _P, _P, _P, _Z, _P],
                            ctypes.c_int),
    "tsv_decode_step_ex": ([_SP, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _OP, _F, _P, _P,
                            _P, _P, _P, _Z, _P], ctypes.c_int),
    "tsv_decode_step_noalloc": ([_SP, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _OP, _F, _P,
                                 _P, _P, _P, _P], ctypes.c_int),
    "tsv_schedule_rows": ([_SP, _I, _P, _P, _I, _I, _P, _I, _P], ctypes.c_int),
    "tsv_step_residency": ([_SP, _I, _P, _P], ctypes.c_int),
    "tsv_decode_step_scheduled": ([_SP, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _OP, _P, _I,
                                   _F, _P, _P, _P, _P, _P, _Z, _P], ctypes.c_int),
}
_TEST_SIGS = {"tsv_debug_exchange_polls": ([_I], ctypes.c_int),
              "tsv_debug_phase_stamps": ([_I, ctypes.c_void_p, ctypes.c_size_t], ctypes.c_int)}


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def _opts(n_recent, group_agg):
    return ctypes.byref(SelectOpts(int(n_recent), int(group_agg)))


def _nbytes(t):
    return t.numel() * t.element_size()


class Library:
    """One loaded copy of the C library; every method marshals its tensors to
    pointers and calls the C function of the same name."""

    def __init__(self, path: str, test_hooks: bool = False):
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; build it with "
                              "`python query_aware_sparse_bbox_amd/build.py` (hipcc, gfx950)")
        self.path = path
        self.lib = ctypes.CDLL(path)
        sigs = dict(_SIGS, **(_TEST_SIGS if test_hooks else {}))
        for name, (args, res) in sigs.items():
            f = getattr(self.lib, name)
            f.argtypes = args
            f.restype = res

    def _call(self, name, *args):
        rc = getattr(self.lib, name)(*args)
        if rc != TSV_OK:
            raise TsvError(name, rc)

    def tsv_version(self) -> int:
        return self.lib.tsv_version()

    def status_string(self, status: int) -> str:
        return self.lib.tsv_status_string(status).decode()

    tsv_status_string = status_string

    def tsv_debug_exchange_polls(self, polls: int) -> int:
        """Testing library only: polls >= 0 sets how long a split row's
        workgroup waits for the others' page scores before scoring the rest
        itself (returns the previous limit); polls < 0 returns the current
        limit."""
        return self.lib.tsv_debug_exchange_polls(int(polls))

    def tsv_debug_phase_stamps(self, kv_dtype: int):
        """Testing library only: the last one-launch step's phase stamps of
        KV type kv_dtype, a uint64 numpy array [8192][8] (slots as in
        include/tsv_testing.h)."""
        import numpy as np

        buf = np.zeros((8192, 8), dtype=np.uint64)
        self._call("tsv_debug_phase_stamps", int(kv_dtype), ctypes.c_void_p(buf.ctypes.data),
                   buf.nbytes)
        return buf

    def tsv_meta_bytes(self, shape) -> int:
        return self.lib.tsv_meta_bytes(ctypes.byref(Shape.of(shape)))

    def tsv_workspace_bytes(self, shape, k_max: int) -> int:
        return self.lib.tsv_workspace_bytes(ctypes.byref(Shape.of(shape)), int(k_max))

    def tsv_decode_step_launches(self, shape, k_max: int, with_append: bool) -> int:
        return self.lib.tsv_decode_step_launches(ctypes.byref(Shape.of(shape)), int(k_max),
                                                 int(bool(with_append)))

    def new_workspace(self, shape, k_max, device="cuda"):
        """A zero-filled workspace of tsv_workspace_bytes(shape, k_max) bytes
        (its first TSV_WORKSPACE_ZERO_BYTES must start at zero; every call
        leaves them so)."""
        import torch
        n = self.tsv_workspace_bytes(shape, k_max)
        if n == 0:
            raise ValueError("shape or k_max not supported")
        return torch.zeros(n, dtype=torch.uint8, device=device)

    def tsv_meta_build(self, shape, k_pool, meta, block_table, seq_lens, stream=None):
        self._call("tsv_meta_build", ctypes.byref(Shape.of(shape)), _ptr(k_pool), _ptr(meta),
                   _ptr(block_table), _ptr(seq_lens), _stream(stream))

    def tsv_meta_append(self, shape, k_new, v_new, k_pool, v_pool, meta, block_table,
                        seq_lens, stream=None):
        self._call("tsv_meta_append", ctypes.byref(Shape.of(shape)), _ptr(k_new), _ptr(v_new),
                   _ptr(k_pool), _ptr(v_pool), _ptr(meta), _ptr(block_table), _ptr(seq_lens),
                   _stream(stream))

    def tsv_select_pages(self, shape, q, meta, block_table, seq_lens, k_max, k_per_seq,
                         n_sink, sel, sel_count, scores_out, workspace, stream=None):
        self._call("tsv_select_pages", ctypes.byref(Shape.of(shape)), _ptr(q), _ptr(meta),
                   _ptr(block_table), _ptr(seq_lens), int(k_max), _ptr(k_per_seq), int(n_sink),
                   _ptr(sel), _ptr(sel_count), _ptr(scores_out), _ptr(workspace),
                   _nbytes(workspace), _stream(stream))

    def tsv_sparse_decode(self, shape, q, k_pool, v_pool, block_table, seq_lens, sel,
                          sel_count, k_max, scale, out, workspace, stream=None):
        self._call("tsv_sparse_decode", ctypes.byref(Shape.of(shape)), _ptr(q), _ptr(k_pool),
                   _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), _ptr(sel),
                   _ptr(sel_count), int(k_max), float(scale), _ptr(out), _ptr(workspace),
                   _nbytes(workspace), _stream(stream))

    def tsv_decode_step(self, shape, q, k_new, v_new, k_pool, v_pool, meta, block_table,
                        seq_lens, k_max, k_per_seq, n_sink, scale, sel, sel_count, scores_out,
                        out, workspace, stream=None):
        self._call("tsv_decode_step", ctypes.byref(Shape.of(shape)), _ptr(q), _ptr(k_new),
                   _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(meta), _ptr(block_table),
                   _ptr(seq_lens), int(k_max), _ptr(k_per_seq), int(n_sink), float(scale),
                   _ptr(sel), _ptr(sel_count), _ptr(scores_out), _ptr(out), _ptr(workspace),
                   _nbytes(workspace), _stream(stream))

    def tsv_select_pages_ex(self, shape, q, meta, block_table, seq_lens, k_max, k_per_seq,
                            n_sink, n_recent, group_agg, sel, sel_count, scores_out, workspace,
                            stream=None):
        self._call("tsv_select_pages_ex", ctypes.byref(Shape.of(shape)), _ptr(q), _ptr(meta),
                   _ptr(block_table), _ptr(seq_lens), int(k_max), _ptr(k_per_seq), int(n_sink),
                   _opts(n_recent, group_agg), _ptr(sel), _ptr(sel_count), _ptr(scores_out),
                   _ptr(workspace), _nbytes(workspace), _stream(stream))

    def tsv_decode_step_ex(self, shape, q, k_new, v_new, k_pool, v_pool, meta, block_table,
                           seq_lens, k_max, k_per_seq, n_sink, n_recent, group_agg, scale, sel,
                           sel_count, scores_out, out, workspace, stream=None):
        self._call("tsv_decode_step_ex", ctypes.byref(Shape.of(shape)), _ptr(q), _ptr(k_new),
                   _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(meta), _ptr(block_table),
                   _ptr(seq_lens), int(k_max), _ptr(k_per_seq), int(n_sink),
                   _opts(n_recent, group_agg), float(scale), _ptr(sel), _ptr(sel_count),
                   _ptr(scores_out), _ptr(out), _ptr(workspace), _nbytes(workspace),
                   _stream(stream))

    def tsv_decode_step_noalloc(self, shape, q, k_new, v_new, k_pool, v_pool, meta,
                                block_table, seq_lens, k_max, k_per_seq, n_sink, n_recent,
                                group_agg, scale, sel, sel_count, scores_out, out, stream=None):
        self._call("tsv_decode_step_noalloc", ctypes.byref(Shape.of(shape)), _ptr(q),
                   _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(meta),
                   _ptr(block_table), _ptr(seq_lens), int(k_max), _ptr(k_per_seq), int(n_sink),
                   _opts(n_recent, group_agg), float(scale), _ptr(sel), _ptr(sel_count),
                   _ptr(scores_out), _ptr(out), _stream(stream))

    def tsv_step_residency(self, shape, k_max: int):
        """(num_cus, per_cu) of the current device for this shape's step."""
        cus, per = ctypes.c_int32(0), ctypes.c_int32(0)
        self._call("tsv_step_residency", ctypes.byref(Shape.of(shape)), int(k_max),
                   ctypes.byref(cus), ctypes.byref(per))
        return cus.value, per.value

    def tsv_schedule_rows(self, shape, k_max, seq_lens, k_per_seq, num_cus, per_cu):
        """The row order (int32 numpy array) for host arrays seq_lens and
        k_per_seq (None allowed) of B entries each."""
        import numpy as np

        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        kp = None if k_per_seq is None else np.ascontiguousarray(k_per_seq, dtype=np.int32)
        if sl.shape != (int(shape.batch),) or (kp is not None and kp.shape != sl.shape):
            raise ValueError("seq_lens / k_per_seq must hold one entry per sequence")
        n = ctypes.c_int32(0)
        args = (ctypes.byref(Shape.of(shape)), int(k_max), ctypes.c_void_p(sl.ctypes.data),
                None if kp is None else ctypes.c_void_p(kp.ctypes.data), int(num_cus),
                int(per_cu))
        self._call("tsv_schedule_rows", *args, None, 0, ctypes.byref(n))
        order = np.empty(n.value, dtype=np.int32)
        self._call("tsv_schedule_rows", *args, ctypes.c_void_p(order.ctypes.data), order.size,
                   ctypes.byref(n))
        return order

    def tsv_decode_step_scheduled(self, shape, q, k_new, v_new, k_pool, v_pool, meta,
                                  block_table, seq_lens, k_max, k_per_seq, n_sink, n_recent,
                                  group_agg, row_order, scale, sel, sel_count, scores_out, out,
                                  workspace, stream=None):
        self._call("tsv_decode_step_scheduled", ctypes.byref(Shape.of(shape)), _ptr(q),
                   _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(meta),
                   _ptr(block_table), _ptr(seq_lens), int(k_max), _ptr(k_per_seq), int(n_sink),
                   _opts(n_recent, group_agg), _ptr(row_order),
                   0 if row_order is None else row_order.numel(), float(scale), _ptr(sel),
                   _ptr(sel_count), _ptr(scores_out), _ptr(out), _ptr(workspace),
                   _nbytes(workspace), _stream(stream))


# the library proper; the module-level functions are its methods
_default = Library(LIB_PATH)
_lib = _default.lib
_testing = None


def testing_library() -> Library:
    """The testing build (libtsv_testhooks.so): the same kernels and entry
    points plus tsv_debug_exchange_polls and tsv_debug_phase_stamps (its
    one-launch step kernels record phase stamps).  Loaded on first use."""
    global _testing
    if _testing is None:
        _testing = Library(TESTHOOKS_PATH, test_hooks=True)
    return _testing


tsv_version = _default.tsv_version
status_string = _default.status_string
tsv_status_string = _default.status_string
tsv_meta_bytes = _default.tsv_meta_bytes
tsv_workspace_bytes = _default.tsv_workspace_bytes
tsv_decode_step_launches = _default.tsv_decode_step_launches
new_workspace = _default.new_workspace
tsv_meta_build = _default.tsv_meta_build
tsv_meta_append = _default.tsv_meta_append
tsv_select_pages = _default.tsv_select_pages
tsv_sparse_decode = _default.tsv_sparse_decode
tsv_decode_step = _default.tsv_decode_step
tsv_select_pages_ex = _default.tsv_select_pages_ex
tsv_decode_step_ex = _default.tsv_decode_step_ex
tsv_decode_step_noalloc = _default.tsv_decode_step_noalloc
tsv_schedule_rows = _default.tsv_schedule_rows
tsv_step_residency = _default.tsv_step_residency
tsv_decode_step_scheduled = _default.tsv_decode_step_scheduled
