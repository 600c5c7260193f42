"""The benchmark's own arithmetic, on the CPU: the algorithmic bytes that the
roofline divides by, and the attention-mass recall of the selection report.

Both are pinned against values that do not reuse their code: bytes counted
token by token from the definition of what a step must move, and recall
values from the softmax written out by hand on small cases, its limits (all
pages kept, none kept), and its invariance under a shift of all logits.
"""
import math
import os
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def counted_bytes(sh, lens, sel, cnt, appends):
    """Bytes of one step counted one token / page / value at a time."""
    e = W.DTYPE_BYTES[sh.kv_dtype]
    P, D = sh.page_size, sh.head_dim
    total = 0
    for b in range(sh.batch):
        n = 0
        while n * P < lens[b]:
            n += 1
        for h in range(sh.num_kv_heads):
            total += n * 2 * D * e                     # min and max row of every page box
            for p in sel[b, h, :cnt[b, h]]:
                for t in range(p * P, p * P + P):      # each valid token's key and value
                    if t < lens[b]:
                        total += 2 * D * e
        total += n * 4                                 # the block-table row
        for _ in range(sh.num_q_heads):
            total += D * 4 + D * 4                     # q read, out written
        if appends:
            for _ in range(sh.num_kv_heads):
                total += 2 * D * e                     # new key and value written
                total += 2 * 2 * D * e                 # the touched box read and written
    return total


@pytest.mark.parametrize("dt,appends", [(W.F16, False), (W.F8, True), (W.F32, True)])
def test_step_bytes_counts_every_token(dt, appends):
    rng = np.random.default_rng(3)
    sh = W.Shape(batch=5, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                 max_pages_per_seq=20, num_phys_pages=100, kv_dtype=dt)
    lens = np.array([1, 16, 17, 300, 250], dtype=np.int64)
    k_max = 6
    sel = np.full((5, 2, k_max), -1, dtype=np.int32)
    cnt = np.zeros((5, 2), dtype=np.int32)
    for b in range(5):
        n = (lens[b] + 15) // 16
        for h in range(2):
            c = min(k_max, n, int(rng.integers(1, k_max + 1)))
            sel[b, h, :c] = np.sort(rng.choice(n, size=c, replace=False))
            cnt[b, h] = c
    wl = SimpleNamespace(shape=sh, steps=[object()] if appends else [])
    got = bench.step_bytes(wl, lens, sel, cnt)
    assert got["total"] == counted_bytes(sh, lens, sel, cnt, appends)
    assert got["total"] == sum(v for k, v in got.items() if k != "total")


def test_recall_by_hand():
    # two pages of two tokens, D = 1: logits are the keys times q = 1
    keys = np.array([[0.0], [math.log(3.0)], [math.log(2.0)], [math.log(4.0)]])
    q = np.array([[1.0]])
    # softmax weights 1, 3, 2, 4 (sum 10): page 0 holds 4/10, page 1 6/10
    assert bench.attention_mass_recall(keys, q, 1.0, 2, [0]) == pytest.approx([0.4], abs=1e-15)
    assert bench.attention_mass_recall(keys, q, 1.0, 2, [1]) == pytest.approx([0.6], abs=1e-15)
    # scale multiplies the logits: weights 1, 9, 4, 16 with scale 2
    assert bench.attention_mass_recall(keys, q, 2.0, 2, [0]) == pytest.approx([10 / 30], abs=1e-15)
    # a ragged last page (one token): pages {0, 1}, {2}
    assert bench.attention_mass_recall(keys[:3], q, 1.0, 2, [1]) == pytest.approx([2 / 6], abs=1e-15)


def test_recall_limits_and_shift_invariance():
    rng = np.random.default_rng(11)
    keys = rng.standard_normal((50, 8)) * 3
    q = rng.standard_normal((4, 8))
    n_pages = (50 + 15) // 16
    assert bench.attention_mass_recall(keys, q, 0.7, 16, range(n_pages)) == pytest.approx([1.0] * 4)
    assert bench.attention_mass_recall(keys, q, 0.7, 16, []) == [0.0] * 4
    # adding a multiple of q's direction to every key shifts each head's
    # logits by a constant when q is one-hot: the softmax does not change
    qh = np.zeros((1, 8))
    qh[0, 2] = 1.0
    shifted = keys.copy()
    shifted[:, 2] += 40.0
    a = bench.attention_mass_recall(keys, qh, 1.0, 16, [1, 3])
    b = bench.attention_mass_recall(shifted, qh, 1.0, 16, [1, 3])
    assert a == pytest.approx(b, rel=1e-12)
    # the kept shares of complementary page sets add to one
    r1 = bench.attention_mass_recall(keys, q, 0.7, 16, [0, 2])
    r2 = bench.attention_mass_recall(keys, q, 0.7, 16, [1, 3])
    assert np.allclose(np.add(r1, r2), 1.0)
