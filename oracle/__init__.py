"""ctypes binding of the CPU oracle (test infrastructure, host arrays only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
use this module; the product path never imports it.  Every function takes and
returns numpy arrays in the layouts of the C library (see tsv_oracle.h) and
raises ``RuntimeError`` when the oracle reports an invalid argument.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size",
                 "max_pages_per_seq", "num_phys_pages", "kv_dtype")]


# The library to load: the built oracle, or (mutation tests only) a copy with
# a planted mistake named by TSV_ORACLE_LIB.
LIB_PATH = os.environ.get("TSV_ORACLE_LIB", _build.LIB)


def _load():
    global _lib
    if _lib is None:
        if LIB_PATH == _build.LIB and not os.path.exists(LIB_PATH):
            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int32
        sig = {
            "tsvo_meta_build": [P, P, P, P, P],
            "tsvo_meta_append": [P, P, P, P, P, P, P, P],
            "tsvo_page_scores": [P, P, P, P, P, I, P],
            "tsvo_select_from_scores": [P, P, P, I, P, I, I, P, P],
            "tsvo_select_pages": [P, P, P, P, P, I, P, I, I, I, P, P, P],
            "tsvo_sparse_decode": [P, P, P, P, P, P, P, P, I, ctypes.c_float, P],
            "tsvo_decode_step": [P, P, P, P, P, P, P, P, P, I, P, I, I, I,
                                 ctypes.c_float, P, P, P, P],
        }
        for name, args in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


# how the G query heads of a KV head combine into the page score
AGG_MAX, AGG_SUM = 0, 1


def shape_of(sh) -> Shape:
    return Shape(sh.batch, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.page_size,
                 sh.max_pages_per_seq, sh.num_phys_pages, sh.kv_dtype)


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} rejected its arguments (rc={rc})")


def meta_bytes_shape(sh):
    return (sh.num_phys_pages, sh.num_kv_heads, 2, sh.head_dim)


def meta_build(sh, k_pool, block_table, seq_lens, meta=None):
    """Bounding box (per-channel min, max) of every page's valid keys."""
    if meta is None:
        meta = np.zeros(meta_bytes_shape(sh), dtype=k_pool.dtype)
    bt, sl = _i32(block_table), _i32(seq_lens)
    _check(_load().tsvo_meta_build(ctypes.byref(shape_of(sh)), _p(k_pool), _p(meta),
                                   _p(bt), _p(sl)), "tsvo_meta_build")
    return meta


def meta_append(sh, k_new, v_new, k_pool, v_pool, meta, block_table, seq_lens):
    """Write the decoded token into its slot and widen its page's box (in place)."""
    bt, sl = _i32(block_table), _i32(seq_lens)
    _check(_load().tsvo_meta_append(ctypes.byref(shape_of(sh)), _p(k_new), _p(v_new),
                                    _p(k_pool), _p(v_pool), _p(meta), _p(bt), _p(sl)),
           "tsvo_meta_append")


def page_scores(sh, q, meta, block_table, seq_lens, group_agg=AGG_MAX):
    """Score of every page (upper bound of q.k over its box, combined over the
    group's query heads by max or sum), [B][Hkv][MP]; NaN past n_b."""
    sc = np.full((sh.batch, sh.num_kv_heads, sh.max_pages_per_seq), np.nan, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    bt, sl = _i32(block_table), _i32(seq_lens)
    _check(_load().tsvo_page_scores(ctypes.byref(shape_of(sh)), _p(q), _p(meta), _p(bt),
                                    _p(sl), group_agg, _p(sc)), "tsvo_page_scores")
    return sc


def select_from_scores(sh, scores, seq_lens, k_max, k_per_seq=None, n_sink=0, n_recent=0):
    sel = np.empty((sh.batch, sh.num_kv_heads, k_max), dtype=np.int32)
    cnt = np.empty((sh.batch, sh.num_kv_heads), dtype=np.int32)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    sl, kp = _i32(seq_lens), _i32(k_per_seq)
    _check(_load().tsvo_select_from_scores(ctypes.byref(shape_of(sh)), _p(scores), _p(sl),
                                           k_max, _p(kp), n_sink, n_recent, _p(sel),
                                           _p(cnt)),
           "tsvo_select_from_scores")
    return sel, cnt


def select_pages(sh, q, meta, block_table, seq_lens, k_max, k_per_seq=None, n_sink=0,
                 n_recent=0, group_agg=AGG_MAX):
    """(sel, sel_count, scores) exactly as the selection rule defines them."""
    sel = np.empty((sh.batch, sh.num_kv_heads, k_max), dtype=np.int32)
    cnt = np.empty((sh.batch, sh.num_kv_heads), dtype=np.int32)
    sc = np.full((sh.batch, sh.num_kv_heads, sh.max_pages_per_seq), np.nan, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    bt, sl, kp = _i32(block_table), _i32(seq_lens), _i32(k_per_seq)
    _check(_load().tsvo_select_pages(ctypes.byref(shape_of(sh)), _p(q), _p(meta), _p(bt),
                                     _p(sl), k_max, _p(kp), n_sink, n_recent, group_agg,
                                     _p(sel), _p(cnt), _p(sc)),
           "tsvo_select_pages")
    return sel, cnt, sc


def sparse_decode(sh, q, k_pool, v_pool, block_table, seq_lens, sel, sel_count, k_max, scale):
    """Softmax attention (double precision) over the selected pages' valid tokens."""
    out = np.empty((sh.batch, sh.num_q_heads, sh.head_dim), dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    bt, sl = _i32(block_table), _i32(seq_lens)
    sel, sel_count = _i32(sel), _i32(sel_count)
    _check(_load().tsvo_sparse_decode(ctypes.byref(shape_of(sh)), _p(q), _p(k_pool),
                                      _p(v_pool), _p(bt), _p(sl), _p(sel), _p(sel_count),
                                      k_max, ctypes.c_float(scale), _p(out)),
           "tsvo_sparse_decode")
    return out


def decode_step(sh, q, k_pool, v_pool, meta, block_table, seq_lens, k_max, scale,
                k_per_seq=None, n_sink=0, k_new=None, v_new=None, n_recent=0,
                group_agg=AGG_MAX):
    """Append (if k_new is given), score, select and attend; pools/meta updated in place."""
    sel = np.empty((sh.batch, sh.num_kv_heads, k_max), dtype=np.int32)
    cnt = np.empty((sh.batch, sh.num_kv_heads), dtype=np.int32)
    sc = np.full((sh.batch, sh.num_kv_heads, sh.max_pages_per_seq), np.nan, dtype=np.float32)
    out = np.empty((sh.batch, sh.num_q_heads, sh.head_dim), dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    bt, sl, kp = _i32(block_table), _i32(seq_lens), _i32(k_per_seq)
    _check(_load().tsvo_decode_step(ctypes.byref(shape_of(sh)), _p(q), _p(k_new), _p(v_new),
                                    _p(k_pool), _p(v_pool), _p(meta), _p(bt), _p(sl), k_max,
                                    _p(kp), n_sink, n_recent, group_agg,
                                    ctypes.c_float(scale), _p(sel), _p(cnt),
                                    _p(sc), _p(out)),
           "tsvo_decode_step")
    return sel, cnt, sc, out
