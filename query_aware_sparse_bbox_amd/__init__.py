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

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtsv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; build it with "
        "`python query_aware_sparse_bbox_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

TSV_F32, TSV_F16, TSV_BF16, TSV_FP8_E4M3, TSV_FP8_E5M2 = 0, 1, 2, 3, 4
TSV_OK, TSV_ERR_INVALID_ARG, TSV_ERR_UNSUPPORTED, TSV_ERR_HIP = 0, -1, -2, -3
TSV_AGG_MAX, TSV_AGG_SUM = 0, 1

EXPORTS = ("tsv_version", "tsv_status_string", "tsv_meta_bytes", "tsv_workspace_bytes",
           "tsv_decode_step_launches", "tsv_meta_build", "tsv_meta_append",
           "tsv_select_pages", "tsv_sparse_decode", "tsv_decode_step",
           "tsv_select_pages_ex", "tsv_decode_step_ex", "tsv_debug_exchange_polls")


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
    "tsv_debug_exchange_polls": ([_I], ctypes.c_int),
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
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


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


def _call(name, *args):
    rc = getattr(_lib, name)(*args)
    if rc != TSV_OK:
        raise TsvError(name, rc)


def tsv_version() -> int:
    return _lib.tsv_version()


def tsv_debug_exchange_polls(polls: int) -> int:
    """Testing hook: polls >= 0 sets how long a split row's workgroup waits for
    the others' page scores before scoring the rest itself (returns the
    previous limit); polls < 0 returns the current limit."""
    return _lib.tsv_debug_exchange_polls(int(polls))


def status_string(status: int) -> str:
    return _lib.tsv_status_string(status).decode()


tsv_status_string = status_string


def tsv_meta_bytes(shape) -> int:
    return _lib.tsv_meta_bytes(ctypes.byref(Shape.of(shape)))


def tsv_workspace_bytes(shape, k_max: int) -> int:
    return _lib.tsv_workspace_bytes(ctypes.byref(Shape.of(shape)), int(k_max))


def tsv_decode_step_launches(shape, k_max: int, with_append: bool) -> int:
    return _lib.tsv_decode_step_launches(ctypes.byref(Shape.of(shape)), int(k_max),
                                         int(bool(with_append)))


def tsv_meta_build(shape, k_pool, meta, block_table, seq_lens, stream=None):
    _call("tsv_meta_build", ctypes.byref(Shape.of(shape)), _ptr(k_pool), _ptr(meta),
          _ptr(block_table), _ptr(seq_lens), _stream(stream))


def tsv_meta_append(shape, k_new, v_new, k_pool, v_pool, meta, block_table, seq_lens,
                    stream=None):
    _call("tsv_meta_append", ctypes.byref(Shape.of(shape)), _ptr(k_new), _ptr(v_new),
          _ptr(k_pool), _ptr(v_pool), _ptr(meta), _ptr(block_table), _ptr(seq_lens),
          _stream(stream))


def tsv_select_pages(shape, q, meta, block_table, seq_lens, k_max, k_per_seq, n_sink,
                     sel, sel_count, scores_out, workspace, stream=None):
    _call("tsv_select_pages", ctypes.byref(Shape.of(shape)), _ptr(q), _ptr(meta),
          _ptr(block_table), _ptr(seq_lens), int(k_max), _ptr(k_per_seq), int(n_sink),
          _ptr(sel), _ptr(sel_count), _ptr(scores_out), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(stream))


def new_workspace(shape, k_max, device="cuda"):
    """A zero-filled workspace of tsv_workspace_bytes(shape, k_max) bytes (its
    first TSV_WORKSPACE_ZERO_BYTES must start at zero; every call leaves them so)."""
    import torch
    n = tsv_workspace_bytes(shape, k_max)
    if n == 0:
        raise ValueError("shape or k_max not supported")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def tsv_sparse_decode(shape, q, k_pool, v_pool, block_table, seq_lens, sel, sel_count,
                      k_max, scale, out, workspace, stream=None):
    _call("tsv_sparse_decode", ctypes.byref(Shape.of(shape)), _ptr(q), _ptr(k_pool),
          _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), _ptr(sel), _ptr(sel_count),
          int(k_max), float(scale), _ptr(out), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(stream))


def tsv_decode_step(shape, q, k_new, v_new, k_pool, v_pool, meta, block_table, seq_lens,
                    k_max, k_per_seq, n_sink, scale, sel, sel_count, scores_out, out,
                    workspace, stream=None):
    _call("tsv_decode_step", ctypes.byref(Shape.of(shape)), _ptr(q), _ptr(k_new),
          _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(meta), _ptr(block_table),
          _ptr(seq_lens), int(k_max), _ptr(k_per_seq), int(n_sink), float(scale),
          _ptr(sel), _ptr(sel_count), _ptr(scores_out), _ptr(out), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(stream))


def _opts(n_recent, group_agg):
    return ctypes.byref(SelectOpts(int(n_recent), int(group_agg)))


def tsv_select_pages_ex(shape, q, meta, block_table, seq_lens, k_max, k_per_seq, n_sink,
                        n_recent, group_agg, sel, sel_count, scores_out, workspace,
                        stream=None):
    _call("tsv_select_pages_ex", ctypes.byref(Shape.of(shape)), _ptr(q), _ptr(meta),
          _ptr(block_table), _ptr(seq_lens), int(k_max), _ptr(k_per_seq), int(n_sink),
          _opts(n_recent, group_agg), _ptr(sel), _ptr(sel_count), _ptr(scores_out),
          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))


def tsv_decode_step_ex(shape, q, k_new, v_new, k_pool, v_pool, meta, block_table, seq_lens,
                       k_max, k_per_seq, n_sink, n_recent, group_agg, scale, sel, sel_count,
                       scores_out, out, workspace, stream=None):
    _call("tsv_decode_step_ex", ctypes.byref(Shape.of(shape)), _ptr(q), _ptr(k_new),
          _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(meta), _ptr(block_table),
          _ptr(seq_lens), int(k_max), _ptr(k_per_seq), int(n_sink),
          _opts(n_recent, group_agg), float(scale), _ptr(sel), _ptr(sel_count),
          _ptr(scores_out), _ptr(out), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(stream))
