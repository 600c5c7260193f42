"""Seeded synthetic decode workloads for query-aware sparse paged decode.

This module only *draws inputs*: clustered keys, values and queries, block
tables, sequence lengths and page budgets, each rounded once to its storage
type.  It computes nothing of the method (no page metadata, no page scores, no
selection, no attention), so the CPU oracle and the HIP path can both be fed
from it without sharing any of the method's arithmetic.

Workload recipe (TinyServe, "Query-Aware Cache Selection for Efficient LLM
Serving", abstract and method-details section): decode over a paged KV cache
whose pages carry bounding boxes of their keys.  The pages name TinyLLaMA,
GPT2-345M and LLaMA-1.3B-scale models but print no tensors, so every input is
synthetic with those models' decode shapes:

* keys: per (sequence, KV head, logical page) a centroid c ~ N(0, 1)^D, each
  token key = c + N(0, 0.5^2)^D;
* values: N(0, 1);
* query of head hq: sum of the centroids of ``hot`` distinct pages of KV head
  hq // G (drawn per query head) + N(0, 0.3^2)^D, kept in fp32;
* keys and values rounded once to the KV dtype (RNE); both sides read the same
  rounded buffers.

Storage conventions: fp32 pools are ``float32`` arrays, fp16 pools
``float16`` arrays, bf16 pools ``uint16`` arrays holding the bf16 bit
patterns and fp8 pools ``uint8`` arrays holding OCP E4M3 ("FN") codes (sign,
4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN only at
magnitude code 0x7F, largest finite 448) or OCP E5M2 codes (sign, 5 exponent
bits with bias 15, 2 mantissa bits, infinities and NaNs at exponent field 31,
largest finite 57344).  fp8 values are stored unscaled (the synthetic keys
and values lie well inside both ranges).  Layouts: pools ``[NP][Hkv][P][D]``, ``q`` ``[B][Hq][D]`` fp32,
``block_table`` ``[B][MP]`` int32, ``seq_lens`` ``[B]`` int32 (length counts
the token being decoded).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

F32, F16, BF16, F8, F8E5 = 0, 1, 2, 3, 4
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16", F8: "fp8e4m3", F8E5: "fp8e5m2"}
DTYPE_BYTES = {F32: 4, F16: 2, BF16: 2, F8: 1, F8E5: 1}
STORAGE_NP = {F32: np.float32, F16: np.float16, BF16: np.uint16, F8: np.uint8, F8E5: np.uint8}


def _e4m3_table() -> np.ndarray:
    """Value of every E4M3 code 0..255 (float64), from the format's definition."""
    c = np.arange(256)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (8.0 + m) * np.exp2(e - 10.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c >= 128, -mag, mag)


def _e5m2_table() -> np.ndarray:
    """Value of every E5M2 code 0..255 (float64), from the format's definition:
    bias 15, 2 mantissa bits, exponent field 31 = infinity (m = 0) or NaN."""
    c = np.arange(256)
    e = (c >> 2) & 0x1F
    m = (c & 3).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -16, (4.0 + m) * np.exp2(e - 17.0))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(c >= 128, -mag, mag)


_E4M3 = _e4m3_table()
_E5M2 = _e5m2_table()


def _round_to_fp8(x: np.ndarray, table: np.ndarray, top: int, nan_code: int) -> np.ndarray:
    """float32 -> fp8 code: nearest finite value (codes 0..top increase with
    the value), ties to the even code, magnitudes beyond the largest finite
    value saturate to it, NaN -> nan_code (sign kept)."""
    pos = table[:top + 1]
    mid = (pos[:-1] + pos[1:]) / 2.0                      # exact in float64
    a = np.abs(x.astype(np.float64))
    lo = np.clip(np.searchsorted(mid, a, side="left"), 0, top)
    # lo = number of midpoints strictly below a: a lies in (mid[lo-1], mid[lo]]
    hi = np.minimum(lo + 1, top)
    tie = (lo < top) & (a == mid[np.minimum(lo, top - 1)])
    code = np.where(tie & (lo % 2 == 1), hi, lo)
    code = np.where(np.isnan(a), nan_code, code).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 7)


@dataclass
class Shape:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    max_pages_per_seq: int
    num_phys_pages: int
    kv_dtype: int

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclass
class AppendStep:
    """One decode step that first appends a token to every sequence."""
    k_new: np.ndarray          # [B][Hkv][D] storage dtype
    v_new: np.ndarray          # [B][Hkv][D] storage dtype
    seq_lens: np.ndarray       # [B] int32, already counting the new token
    k_per_seq: Optional[np.ndarray]
    q: np.ndarray              # [B][Hq][D] fp32


@dataclass
class Workload:
    name: str
    shape: Shape
    k_pool: np.ndarray
    v_pool: np.ndarray
    q: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    k_max: int
    k_per_seq: Optional[np.ndarray]
    n_sink: int
    scale: float
    steps: list = field(default_factory=list)   # list[AppendStep]

    @property
    def n_pages(self) -> np.ndarray:
        P = self.shape.page_size
        return (self.seq_lens.astype(np.int64) + P - 1) // P


# ----------------------------------------------------------------------------
# storage rounding (input preparation only)
# ----------------------------------------------------------------------------

def to_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float data once, to nearest-even, into the KV storage type."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == F32:
        return x.copy()
    if dtype == F16:
        return x.astype(np.float16)
    if dtype == BF16:
        # RNE on the bit pattern; cannot wrap for finite values or default NaNs
        u = x.view(np.uint32)
        u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return u.astype(np.uint16)
    if dtype == F8:
        return _round_to_fp8(x, _E4M3, 0x7E, 0x7F)
    if dtype == F8E5:
        return _round_to_fp8(x, _E5M2, 0x7B, 0x7F)
    raise ValueError(f"unknown kv dtype {dtype}")


def storage_to_f32(a: np.ndarray, dtype: int) -> np.ndarray:
    """Exact widening of stored KV values to float32 (for test-side formulas)."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32)
    if dtype == F16:
        return np.asarray(a, dtype=np.float16).astype(np.float32)
    if dtype == BF16:
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    if dtype in (F8, F8E5):
        t = _E4M3 if dtype == F8 else _E5M2
        return t[np.asarray(a, dtype=np.uint8)].astype(np.float32)
    raise ValueError(f"unknown kv dtype {dtype}")


# ----------------------------------------------------------------------------
# generator
# ----------------------------------------------------------------------------

@dataclass
class Spec:
    """Shape and distribution of one synthetic decode workload."""
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: int
    context: int = 1024                 # fixed length when lens_range is None
    lens_range: Optional[tuple] = None  # (lo, hi) inclusive, per-sequence uniform
    budget: tuple = ("fixed", 8)        # ("fixed", K) | ("fraction", num, den) | ("ragged", cap, den)
    n_sink: int = 0
    hot: int = 2                        # hot pages per query head
    hot_from: int = 0                   # first logical page hot pages may come from
    layout: str = "contiguous"          # contiguous | permuted | shared_shuffled
    append_steps: int = 0               # decode steps that append one token each
    centroid_sigma: float = 1.0
    noise_sigma: float = 0.5
    query_sigma: float = 0.3


def _budget(spec: Spec, n_pages: np.ndarray):
    """Page budget K_b per sequence and the row width k_max."""
    kind = spec.budget[0]
    if kind == "fixed":
        k = int(spec.budget[1])
        return k, None
    if kind == "fraction":
        num, den = spec.budget[1], spec.budget[2]
        per = np.maximum(1, (n_pages * num) // den).astype(np.int32)
        if np.all(per == per[0]):
            return int(per[0]), None
        return int(per.max()), per
    if kind == "ragged":
        cap, den = spec.budget[1], spec.budget[2]
        per = np.minimum(cap, np.maximum(1, n_pages // den)).astype(np.int32)
        return int(cap), per
    raise ValueError(kind)


def _draw_queries(rng, spec: Spec, centroids, n_pages, G):
    B, Hq, D = spec.batch, spec.num_q_heads, spec.head_dim
    q = np.empty((B, Hq, D), dtype=np.float32)
    for b in range(B):
        nb = int(n_pages[b])
        lo = min(spec.hot_from, max(nb - 1, 0))
        pool = np.arange(lo, nb)
        for hq in range(Hq):
            h = hq // G
            k = min(spec.hot, len(pool))
            hot = rng.choice(pool, size=k, replace=False)
            acc = centroids[b][h, hot, :].astype(np.float64).sum(axis=0)
            acc += spec.query_sigma * rng.standard_normal(D)
            q[b, hq] = acc.astype(np.float32)
    return q


def generate(spec: Spec, seed: int) -> Workload:
    """Draw one workload from ``spec`` with ``numpy.random.Generator(PCG64(seed))``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, Hq, Hkv, D, P = (spec.batch, spec.num_q_heads, spec.num_kv_heads,
                        spec.head_dim, spec.page_size)
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    if spec.lens_range is None:
        lens0 = np.full(B, spec.context, dtype=np.int64)
    else:
        lo, hi = spec.lens_range
        lens0 = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    S = spec.append_steps
    # lengths at the first decode step: with appends the first step adds one token
    first_lens = lens0 + (1 if S > 0 else 0)
    cap_tokens = lens0 + S                      # tokens the pool must hold
    cap_pages = (cap_tokens + P - 1) // P
    MP = int(cap_pages.max())
    if spec.layout in ("contiguous", "permuted"):
        NP = B * MP
        if spec.layout == "contiguous":
            bt = (np.arange(B, dtype=np.int64)[:, None] * MP + np.arange(MP)[None, :])
        else:
            bt = rng.permutation(NP).reshape(B, MP)
        bt = bt.astype(np.int32)
    elif spec.layout == "shared_shuffled":
        NP = int(cap_pages.sum())
        perm = rng.permutation(NP).astype(np.int32)
        bt = np.zeros((B, MP), dtype=np.int32)
        off = 0
        for b in range(B):
            c = int(cap_pages[b])
            bt[b, :c] = perm[off:off + c]
            off += c
    else:
        raise ValueError(spec.layout)

    dt = spec.kv_dtype
    k_pool = np.zeros((NP, Hkv, P, D), dtype=STORAGE_NP[dt])
    v_pool = np.zeros((NP, Hkv, P, D), dtype=STORAGE_NP[dt])
    # every sequence draws from its own child stream, so the result does not
    # depend on how many threads fill the pool
    seq_seeds = np.random.SeedSequence(seed).spawn(B)
    centroids = [None] * B

    def fill(b):
        r = np.random.Generator(np.random.PCG64(seq_seeds[b]))
        # centroids for every page the sequence will ever own (appends that
        # open a page use that page's own fresh centroid)
        nc = int(cap_pages[b])
        c = spec.centroid_sigma * r.standard_normal((Hkv, nc, D), dtype=np.float32)
        centroids[b] = c
        npre = int((lens0[b] + P - 1) // P)        # pages holding the prefix
        keys = r.standard_normal((Hkv, npre, P, D), dtype=np.float32)
        keys *= np.float32(spec.noise_sigma)
        keys += c[:, :npre, None, :]
        vals = r.standard_normal((Hkv, npre, P, D), dtype=np.float32)
        phys = bt[b, :npre]
        k_pool[phys] = to_storage(keys, dt).transpose(1, 0, 2, 3)
        v_pool[phys] = to_storage(vals, dt).transpose(1, 0, 2, 3)

    workers = max(1, min(8, os.cpu_count() or 1, B))
    if workers == 1:
        for b in range(B):
            fill(b)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(B)))

    shape = Shape(B, Hq, Hkv, D, P, MP, NP, dt)
    n_first = (first_lens + P - 1) // P
    k_max, k_per = _budget(spec, n_first)
    q0 = _draw_queries(rng, spec, centroids, n_first, G)
    wl = Workload(spec.name, shape, k_pool, v_pool, q0, bt,
                  first_lens.astype(np.int32), k_max, k_per, spec.n_sink,
                  float(np.float32(1.0 / math.sqrt(D))))
    if S > 0:
        # the prefix is lens0; step i appends token index lens0 + i
        lens = lens0.copy()
        for i in range(S):
            pos = lens                                # 0-based index of the new token
            pg = pos // P
            kn = np.empty((B, Hkv, D), dtype=np.float32)
            for b in range(B):
                kn[b] = centroids[b][:, int(pg[b]), :] + np.float32(spec.noise_sigma) * \
                    rng.standard_normal((Hkv, D), dtype=np.float32)
            vn = rng.standard_normal((B, Hkv, D), dtype=np.float32)
            lens = lens + 1
            n_now = (lens + P - 1) // P
            _, kp = _budget(spec, n_now)
            qi = q0 if i == 0 else _draw_queries(rng, spec, centroids, n_now, G)
            wl.steps.append(AppendStep(to_storage(kn, dt), to_storage(vn, dt),
                                       lens.astype(np.int32), kp, qi))
        wl.k_per_seq = wl.steps[0].k_per_seq
    return wl


# ----------------------------------------------------------------------------
# the five decode configurations
# ----------------------------------------------------------------------------

SPECS = {
    # tiny MHA, fp32 KV, 64 pages, top-8
    "tiny": Spec("tiny", 1, 4, 4, 64, 16, F32, context=1024,
                 budget=("fixed", 8), hot=2),
    # TinyLLaMA-1.1B-shaped GQA decode, bf16 KV, budget 25% of pages
    "tinyllama": Spec("tinyllama", 16, 32, 4, 64, 16, BF16, context=4096,
                      budget=("fraction", 1, 4), hot=4),
    # GPT2-345M-shaped MHA decode, fp16 KV, top-16, pool randomly permuted
    "gpt2": Spec("gpt2", 32, 16, 16, 64, 16, F16, context=1024,
                 budget=("fixed", 16), hot=2, layout="permuted"),
    # LLaMA-1.3B-shaped 32K context, bf16 KV, budget 1/16 incl. one sink page
    "llama_long": Spec("llama_long", 8, 32, 32, 64, 32, BF16, context=32768,
                       budget=("fraction", 1, 16), n_sink=1, hot=8, hot_from=1),
    # ragged serving mix: GQA 4, D=128, fp16, shared shuffled pool, appends
    "ragged": Spec("ragged", 64, 32, 8, 128, 16, F16, lens_range=(512, 16384),
                   budget=("ragged", 64, 5), hot=4, layout="shared_shuffled",
                   append_steps=1),
}

CONFIG_ORDER = ["tiny", "tinyllama", "gpt2", "llama_long", "ragged"]
SEEDS = {name: 1000 + i + 1 for i, name in enumerate(CONFIG_ORDER)}


def spec(name: str, **overrides) -> Spec:
    return replace(SPECS[name], **overrides)


def make(name: str, seed: Optional[int] = None, **overrides) -> Workload:
    """Workload ``name`` (optionally reshaped by ``overrides``) at its seed."""
    s = spec(name, **overrides)
    return generate(s, SEEDS[name] if seed is None else seed)


# ----------------------------------------------------------------------------
# input variants used by tests
# ----------------------------------------------------------------------------

def poison_unused(wl: Workload, steps_ahead: int = 0) -> None:
    """Fill every pool slot no valid token occupies with NaN (in place).

    Slots at or past each sequence's length, and pages no sequence owns, are
    set to NaN so that any read of them shows up in the results.  With
    ``steps_ahead`` > 0 the slots the next appends will fill are kept as NaN
    too (the appends overwrite them).
    """
    dt = wl.shape.kv_dtype
    nan = to_storage(np.array([np.nan], dtype=np.float32), dt)[0]
    P = wl.shape.page_size
    used = np.zeros((wl.shape.num_phys_pages, P), dtype=bool)
    lens = wl.seq_lens.astype(np.int64)
    if wl.steps:
        lens = wl.steps[0].seq_lens.astype(np.int64) - 1   # before the first append
    for b in range(wl.shape.batch):
        L = int(lens[b])
        n = (L + P - 1) // P
        for p in range(n):
            v = min(P, L - p * P)
            used[wl.block_table[b, p], :v] = True
    mask = ~used
    kp = wl.k_pool.reshape(wl.shape.num_phys_pages, wl.shape.num_kv_heads, P, -1)
    vp = wl.v_pool.reshape(wl.shape.num_phys_pages, wl.shape.num_kv_heads, P, -1)
    idx = np.nonzero(mask)
    kp[idx[0], :, idx[1], :] = nan
    vp[idx[0], :, idx[1], :] = nan


def tie_heavy(seed: int, batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
              page_size=16, context=200, kv_dtype=BF16, value_range=3,
              k_max=5, n_sink=0, layout="permuted") -> Workload:
    """Small-integer keys and queries: every product and partial sum is exact.

    With all values in [-value_range, value_range] and small D, page scores are
    exact integers whatever the summation order, so equal scores are common and
    only the tie rule decides the selection.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, Hq, Hkv, D, P = batch, num_q_heads, num_kv_heads, head_dim, page_size
    MP = (context + P - 1) // P
    NP = B * MP
    bt = (rng.permutation(NP) if layout == "permuted" else np.arange(NP)).reshape(B, MP)
    k = rng.integers(-value_range, value_range + 1, size=(NP, Hkv, P, D)).astype(np.float32)
    v = rng.integers(-value_range, value_range + 1, size=(NP, Hkv, P, D)).astype(np.float32)
    q = rng.integers(-value_range, value_range + 1, size=(B, Hq, D)).astype(np.float32)
    shape = Shape(B, Hq, Hkv, D, P, MP, NP, kv_dtype)
    return Workload("tie_heavy", shape, to_storage(k, kv_dtype), to_storage(v, kv_dtype),
                    q, bt.astype(np.int32), np.full(B, context, dtype=np.int32),
                    k_max, None, n_sink, float(np.float32(1.0 / math.sqrt(D))))
