"""The longest-first row schedule of the one-launch step, on the CPU.

tsv_schedule_rows is host code: from the host copy of the sequence lengths
and budgets it ranks the step's (sequence, KV head) rows by the bytes each one
reads and writes the order in which the step's workgroups take them.  The
order only changes which workgroup runs which row (the GPU tests check that
the results are bitwise the same); these tests check what the order itself
promises: every row exactly once, idle slots only inside the first wave, at
most per_cu rows per CU in that wave, the heaviest rows first, and the
balance of the first wave -- optimal where two rows share each CU (sorted
pairing, checked against every pairing of small cases) and within the
4/3 - 1/(3m) bound of longest-first list scheduling with at most three jobs
per machine (Kellerer and Woeginger) against an exhaustive optimum.
"""
import ctypes
import itertools

import numpy as np
import pytest

import workloads as W

F16 = W.F16


@pytest.fixture(scope="module")
def T():
    import query_aware_sparse_bbox_amd as m
    return m


def shape(B, Hkv=2, G=4, D=128, P=16, MP=256, dt=F16):
    return W.Shape(batch=B, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D, page_size=P,
                   max_pages_per_seq=MP, num_phys_pages=B * MP, kv_dtype=dt)


def row_bytes(sh, k_max, lens, kps):
    """Bytes a row reads, as the schedule ranks rows: every page box (min and
    max rows), a full budget of full pages of keys and values, the block-table
    row; the same for the KV heads of one sequence."""
    e = {W.F32: 4, W.F16: 2, W.BF16: 2, W.F8: 1, W.F8E5: 1}[sh.kv_dtype]
    D, P = sh.head_dim, sh.page_size
    lens = np.clip(np.asarray(lens, dtype=np.int64), 0, sh.max_pages_per_seq * P)
    n = (lens + P - 1) // P
    kb = np.full_like(n, k_max) if kps is None else np.asarray(kps, dtype=np.int64)
    kb = np.minimum(n, np.clip(kb, 1, k_max))
    w = 2 * D * e * n + 2 * D * e * P * kb + 4 * n
    return np.repeat(w.astype(np.float64), sh.num_kv_heads)


def cu_rows(order, C, wave):
    """Rows of each CU in the first wave (workgroup j*C + c runs on CU c)."""
    rows = [[] for _ in range(C)]
    for i in range(wave):
        if order[i] >= 0:
            rows[i % C].append(int(order[i]))
    return rows


def first_wave(order, units, C, per):
    first = min(units, C * per)
    return len(order) - (units - first)


@pytest.mark.parametrize("seed", range(12))
def test_every_row_once_and_the_wave_shape(T, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 90))
    Hkv = int(rng.choice([1, 2, 8]))
    sh = shape(B, Hkv=Hkv, MP=64)
    lens = rng.integers(0, 64 * 16 + 1, size=B)
    kps = rng.integers(-3, 40, size=B) if seed % 2 else None
    k_max = int(rng.integers(1, 33))
    C = int(rng.choice([1, 3, 8, 32, 256]))
    per = int(rng.integers(1, 5))
    order = T.tsv_schedule_rows(sh, k_max, lens, kps, C, per)
    U = B * Hkv
    assert sorted(order[order >= 0].tolist()) == list(range(U))
    assert np.all((order >= 0) | (order == -1))
    assert len(order) <= max(U, C * per)
    wave = first_wave(order, U, C, per)
    assert np.all(order[wave:] >= 0), "idle slots only inside the first wave"
    rows = cu_rows(order, C, wave)
    assert max(len(r) for r in rows) <= per
    assert sum(len(r) for r in rows) == min(U, C * per)
    w = row_bytes(sh, k_max, lens, kps)
    # the first wave holds the heaviest rows, the rest follow heaviest first
    # (equal weights: lower row first)
    firsts = {u for r in rows for u in r}
    later = order[wave:]
    if len(later):
        assert min(w[u] for u in firsts) >= w[later].max()
        key = [(-w[u], u) for u in later]
        assert key == sorted(key)


def test_one_row_per_cu_is_descending(T):
    sh = shape(40, Hkv=1)
    lens = np.arange(40) * 37 % 2000 + 1
    order = T.tsv_schedule_rows(sh, 8, lens, None, 64, 2)
    w = row_bytes(sh, 8, lens, None)
    assert len(order) == 40  # no idle slot after the last row
    key = [(-w[u], u) for u in order]
    assert key == sorted(key)


def test_equal_rows_keep_their_order(T):
    sh = shape(10, Hkv=8)
    order = T.tsv_schedule_rows(sh, 16, np.full(10, 700), None, 256, 2)
    assert order.tolist() == list(range(80))


def test_longer_sequences_go_first(T):
    sh = shape(6, Hkv=2)
    lens = np.array([100, 4000, 50, 2500, 3000, 10])
    order = T.tsv_schedule_rows(sh, 1000, lens, None, 256, 1)
    seqs = [u // 2 for u in order]
    assert seqs == [1, 1, 4, 4, 3, 3, 0, 0, 2, 2, 5, 5]


def best_pairing(w):
    """Smallest possible largest pair sum over every perfect matching."""
    best = np.inf

    def rec(rest, worst):
        nonlocal best
        if worst >= best:
            return
        if not rest:
            best = worst
            return
        a = rest[0]
        for i in range(1, len(rest)):
            rec(rest[1:i] + rest[i + 1:], max(worst, w[a] + w[rest[i]]))

    rec(list(range(len(w))), 0.0)
    return best


@pytest.mark.parametrize("seed", range(8))
def test_two_rows_per_cu_is_the_optimal_pairing(T, seed):
    rng = np.random.default_rng(100 + seed)
    C = int(rng.integers(2, 6))
    sh = shape(2 * C, Hkv=1)
    lens = rng.integers(1, 4000, size=2 * C)
    order = T.tsv_schedule_rows(sh, 64, lens, None, C, 2)
    w = row_bytes(sh, 64, lens, None)
    rows = cu_rows(order, C, len(order))
    assert all(len(r) == 2 for r in rows)
    worst = max(w[r].sum() for r in rows)
    assert worst == best_pairing(w)
    # heaviest with lightest: the c-th heaviest weight pairs with the c-th
    # lightest (compared as weights: rows of equal weight are interchangeable)
    ws = np.sort(w)[::-1]
    pairs = sorted(tuple(sorted(w[r].tolist())) for r in rows)
    assert pairs == sorted(tuple(sorted((ws[c], ws[2 * C - 1 - c]))) for c in range(C))


def best_partition(w, C, per):
    """Smallest possible largest CU load with at most per rows per CU."""
    best = np.inf
    order = np.argsort(-w)

    def rec(i, loads, counts):
        nonlocal best
        if max(loads) >= best:
            return
        if i == len(order):
            best = max(loads)
            return
        seen = set()
        for c in range(C):
            if counts[c] < per and (loads[c], counts[c]) not in seen:
                seen.add((loads[c], counts[c]))
                loads[c] += w[order[i]]
                counts[c] += 1
                rec(i + 1, loads, counts)
                loads[c] -= w[order[i]]
                counts[c] -= 1

    rec(0, [0.0] * C, [0] * C)
    return best


@pytest.mark.parametrize("seed", range(10))
def test_three_rows_per_cu_within_the_lpt_bound(T, seed):
    rng = np.random.default_rng(200 + seed)
    C = int(rng.integers(2, 4))
    U = int(rng.integers(C + 1, 3 * C + 1))
    sh = shape(U, Hkv=1)
    lens = rng.integers(1, 4000, size=U)
    order = T.tsv_schedule_rows(sh, 64, lens, None, C, 3)
    w = row_bytes(sh, 64, lens, None)
    rows = cu_rows(order, C, len(order))
    assert max(len(r) for r in rows) <= 3
    worst = max(w[r].sum() for r in rows if r)
    opt = best_partition(w, C, 3)
    assert worst <= (4 / 3 - 1 / (3 * C)) * opt + 1e-9


def test_ragged_mix_first_wave_balance(T):
    """The ragged serving mix (64 sequences of 512-16384 tokens, 8 KV heads,
    budgets min(64, pages/5)) on 256 CUs of two rows each: every CU gets two
    rows, and the heaviest CU holds at most 10% more than the mean (the
    rows' own spread allows no better pairing)."""
    wl = W.make("ragged")
    st = wl.steps[0]
    order = T.tsv_schedule_rows(wl.shape, wl.k_max, st.seq_lens, st.k_per_seq, 256, 2)
    assert len(order) == 512 and np.all(order >= 0)
    w = row_bytes(wl.shape, wl.k_max, st.seq_lens, st.k_per_seq)
    loads = np.array([w[r].sum() for r in cu_rows(order, 256, 512)])
    assert loads.max() <= 1.10 * loads.mean()
    # the identity order puts sequences b and b + 32 together: far worse
    ident = np.array([w[[c, c + 256]].sum() for c in range(256)])
    assert ident.max() > 1.25 * loads.mean()


def test_length_query_and_capacity(T):
    sh = shape(20, Hkv=2)
    lens = np.arange(20) * 100 + 1
    L = T._lib
    s = T.Shape.of(sh)
    lens32 = np.ascontiguousarray(lens, dtype=np.int32)
    n = ctypes.c_int32(-1)
    p = ctypes.c_void_p(lens32.ctypes.data)
    assert L.tsv_schedule_rows(ctypes.byref(s), 8, p, None, 16, 2, None, 0, ctypes.byref(n)) == 0
    assert n.value == len(T.tsv_schedule_rows(sh, 8, lens, None, 16, 2))
    out = np.zeros(n.value, dtype=np.int32)
    o = ctypes.c_void_p(out.ctypes.data)
    assert L.tsv_schedule_rows(ctypes.byref(s), 8, p, None, 16, 2, o, n.value - 1,
                               ctypes.byref(n)) == -1
    for args in [(8, None, None, 16, 2), (8, p, None, 0, 2), (8, p, None, 16, 0),
                 (0, p, None, 16, 2)]:
        k, lp, kp, cus, per = args
        assert L.tsv_schedule_rows(ctypes.byref(s), k, lp, kp, cus, per, o, n.value,
                                   ctypes.byref(n)) == -1
    assert L.tsv_schedule_rows(ctypes.byref(s), 8, p, None, 16, 2, o, n.value, None) == -1
