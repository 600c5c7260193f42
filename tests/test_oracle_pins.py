"""Pins of the CPU oracle to facts fixed outside the oracle itself.

The pages (TinyServe, "Query-Aware Cache Selection for Efficient LLM
Serving": abstract; method details, key design) print no worked example, so
the oracle is pinned to what the mathematics of the method fixes:

* page score = the largest q.k any point of the page's bounding box reaches
  (closed form: the maximum over the box's 2^D corners), within the fp32
  rounding bound of one product plus the summation tree's depth;
* the score bounds every true q.k inside the page (the property that makes
  the box a safe relevance estimate);
* the fixed fp32 summation order, through hand-derived values that differ
  under any other order;
* selection = the unique subset every member of which beats every
  non-member under (score desc, lower page first), found by exhaustive search;
* with every page selected, attention equals dense softmax attention computed
  independently in float64; with scale 0 it is the plain mean of V; a single
  token returns its value row;
* the box is the tightest: every key lies inside, every face is attained.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O
import workloads as W

U = 2.0 ** -24  # unit roundoff of fp32


# ----------------------------------------------------------------------------
# helpers that build small inputs by hand
# ----------------------------------------------------------------------------

def make_wl(keys, vals, q, lens, page_size, dtype=W.F32, block_table=None):
    """Workload from logical keys/vals [B][Hkv][T][D] (float) and q [B][Hq][D]."""
    keys = np.asarray(keys, dtype=np.float32)
    vals = np.asarray(vals, dtype=np.float32)
    B, Hkv, T, D = keys.shape
    Hq = q.shape[1]
    P = page_size
    MP = (T + P - 1) // P
    NP = B * MP
    if block_table is None:
        block_table = np.arange(NP, dtype=np.int32).reshape(B, MP)
    kp = np.zeros((NP, Hkv, P, D), dtype=np.float32)
    vp = np.zeros((NP, Hkv, P, D), dtype=np.float32)
    pad = MP * P - T
    kpad = np.concatenate([keys, np.zeros((B, Hkv, pad, D), np.float32)], axis=2)
    vpad = np.concatenate([vals, np.zeros((B, Hkv, pad, D), np.float32)], axis=2)
    for b in range(B):
        for p in range(MP):
            kp[block_table[b, p]] = kpad[b, :, p * P:(p + 1) * P]
            vp[block_table[b, p]] = vpad[b, :, p * P:(p + 1) * P]
    sh = W.Shape(B, Hq, Hkv, D, P, MP, NP, dtype)
    return W.Workload("hand", sh, W.to_storage(kp, dtype), W.to_storage(vp, dtype),
                      np.ascontiguousarray(q, dtype=np.float32),
                      np.ascontiguousarray(block_table, dtype=np.int32),
                      np.asarray(lens, dtype=np.int32), MP, None, 0,
                      float(np.float32(1.0 / math.sqrt(D))))


def scores_of(wl):
    sh = wl.shape
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    return meta, O.page_scores(sh, wl.q, meta, wl.block_table, wl.seq_lens)


def corner_max(q, mn, mx):
    """max over the 2^D corners x of the box [mn, mx] of q.x, in float64."""
    D = len(q)
    bits = ((np.arange(2 ** D)[:, None] >> np.arange(D)[None, :]) & 1).astype(bool)
    X = np.where(bits, mx[None, :].astype(np.float64), mn[None, :].astype(np.float64))
    return float((X @ q.astype(np.float64)).max())


def tree_bound(q, mn, mx):
    """Rounding bound: one product rounding plus log2(D) tree levels, first order."""
    D = len(q)
    t = np.maximum(q.astype(np.float64) * mn, q.astype(np.float64) * mx)
    return (1 + math.log2(D)) * U * np.abs(t).sum() * 1.0001 + 1e-45


def page_pool_rows(wl, b, h, p):
    """Valid keys of logical page p of sequence b, KV head h, as float64 rows."""
    sh = wl.shape
    P = sh.page_size
    v = min(P, int(wl.seq_lens[b]) - p * P)
    phys = wl.block_table[b, p]
    k = W.storage_to_f32(wl.k_pool[phys, h, :v], sh.kv_dtype).astype(np.float64)
    return k


# ----------------------------------------------------------------------------
# storage decoding: every finite fp16 / bf16 pattern
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_decoder_every_finite_pattern(dtype):
    """Score of a one-token page with q = 1 is the token's value (D = 1)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if dtype == W.F16:
        vals = bits.view(np.float16).astype(np.float32)
    else:
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(vals)
    bits, vals = bits[keep], vals[keep]
    n = len(bits)
    sh = W.Shape(1, 1, 1, 1, 1, n, n, dtype)
    kpool = bits.reshape(n, 1, 1, 1).copy()
    if dtype == W.F16:
        kpool = kpool.view(np.float16)
    bt = np.arange(n, dtype=np.int32).reshape(1, n)
    lens = np.array([n], dtype=np.int32)
    meta = O.meta_build(sh, kpool, bt, lens)
    sc = O.page_scores(sh, np.ones((1, 1, 1), np.float32), meta, bt, lens)[0, 0]
    expect = vals.copy()
    expect[expect == 0] = 0.0  # -0 is stored as +0
    assert np.array_equal(sc.view(np.uint32), expect.view(np.uint32))


FP8 = [  # (KV type, torch type name, finite codes, rounding range, saturating code)
    (W.F8, "float8_e4m3fn", 254, 464, 0x7E),
    (W.F8E5, "float8_e5m2", 248, 61440, 0x7B),
]


@pytest.mark.parametrize("dt,tname,nfinite,lim,top", FP8, ids=["e4m3", "e5m2"])
def test_fp8_decoder_every_finite_pattern(dt, tname, nfinite, lim, top):
    """Every finite OCP fp8 code decodes to torch's value of it (D = 1)."""
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes.copy()).view(getattr(torch, tname)).float().numpy()
    keep = np.isfinite(lib)
    assert keep.sum() == nfinite
    codes, vals = codes[keep], lib[keep]
    n = len(codes)
    sh = W.Shape(1, 1, 1, 1, 1, n, n, dt)
    bt = np.arange(n, dtype=np.int32).reshape(1, n)
    lens = np.array([n], dtype=np.int32)
    meta = O.meta_build(sh, codes.reshape(n, 1, 1, 1), bt, lens)
    sc = O.page_scores(sh, np.ones((1, 1, 1), np.float32), meta, bt, lens)[0, 0]
    expect = vals.copy()
    expect[expect == 0] = 0.0
    assert np.array_equal(sc.view(np.uint32), expect.view(np.uint32))
    # the generator's widening table agrees with the library too
    back = W.storage_to_f32(np.arange(256, dtype=np.uint8), dt)
    assert np.array_equal(back[keep].view(np.uint32), lib[keep].view(np.uint32))


@pytest.mark.parametrize("dt,tname,nfinite,lim,top", FP8, ids=["e4m3", "e5m2"])
def test_fp8_rounding_is_nearest_even(dt, tname, nfinite, lim, top):
    """Input rounding to fp8: torch's conversion inside the finite range
    (every midpoint included), saturation to the largest finite value outside
    it."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    grid = W.storage_to_f32(np.arange(top + 1, dtype=np.uint8), dt).astype(np.float64)
    mids = (grid[:-1] + grid[1:]) / 2
    x = np.concatenate([rng.normal(0, 1, 50000), rng.normal(0, lim / 12, 50000),
                        rng.normal(0, 0.01, 20000), mids, -mids,
                        np.nextafter(mids, 0), np.nextafter(mids, 1e9)]).astype(np.float32)
    x = x[np.abs(x) < lim]
    got = W.to_storage(x, dt)
    lib = torch.from_numpy(x).to(getattr(torch, tname)).view(torch.uint8).numpy()
    assert np.array_equal(got, lib)
    # brute force: the stored value is a nearest grid point
    v = W.storage_to_f32(got, dt).astype(np.float64)
    sgrid = np.concatenate([-grid[::-1], grid])
    dist = np.abs(x.astype(np.float64)[:, None] - sgrid[None, :]).min(axis=1)
    assert np.array_equal(np.abs(x - v), dist)
    big = np.array([lim, lim + 1, 1e30, -1e30], np.float32)
    assert W.to_storage(big, dt).tolist() == [top, top, top, top | 0x80]


# ----------------------------------------------------------------------------
# page score: closed form and bound
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("D,G,P", [(2, 1, 3), (4, 2, 5), (8, 3, 4), (16, 2, 7), (16, 1, 1)])
def test_score_equals_box_corner_maximum(D, G, P):
    rng = np.random.default_rng(7 + D + G)
    B, Hkv, T = 2, 2, 5 * P - 2
    keys = rng.normal(size=(B, Hkv, T, D)) * rng.uniform(0.1, 3.0, size=(1, 1, 1, D))
    q = rng.normal(size=(B, Hkv * G, D)) * 2
    wl = make_wl(keys, rng.normal(size=(B, Hkv, T, D)), q, [T, T - P + 1], P)
    meta, sc = scores_of(wl)
    for b in range(B):
        n = -(-int(wl.seq_lens[b]) // P)
        for h in range(Hkv):
            for p in range(n):
                phys = wl.block_table[b, p]
                mn = meta[phys, h, 0].astype(np.float64)
                mx = meta[phys, h, 1].astype(np.float64)
                exact = [corner_max(wl.q[b, h * G + g], mn, mx) for g in range(G)]
                g_best = int(np.argmax(exact))
                bound = max(tree_bound(wl.q[b, h * G + g], mn, mx) for g in range(G))
                assert abs(sc[b, h, p] - max(exact)) <= bound, (b, h, p, g_best)


def test_score_bounds_every_key_in_the_page():
    """Check (b): score >= max over tokens and group heads of q.k (minus rounding)."""
    wl = W.make("ragged", batch=3, lens_range=(40, 300), append_steps=0,
                num_q_heads=8, num_kv_heads=2)
    sh = wl.shape
    G = sh.group
    meta, sc = scores_of(wl)
    P = sh.page_size
    for b in range(sh.batch):
        n = -(-int(wl.seq_lens[b]) // P)
        for h in range(sh.num_kv_heads):
            for p in range(n):
                k = page_pool_rows(wl, b, h, p)
                qg = wl.q[b, h * G:(h + 1) * G].astype(np.float64)
                true_max = (k @ qg.T).max()
                phys = wl.block_table[b, p]
                mn = W.storage_to_f32(meta[phys, h, 0], sh.kv_dtype).astype(np.float64)
                mx = W.storage_to_f32(meta[phys, h, 1], sh.kv_dtype).astype(np.float64)
                bound = max(tree_bound(qg[g], mn, mx) for g in range(G))
                assert sc[b, h, p] >= true_max - bound


def test_one_token_page_score_is_rounded_dot():
    """A one-token page's box is a point: score = q.k within the rounding bound."""
    rng = np.random.default_rng(3)
    D = 64
    keys = rng.normal(size=(1, 1, 1, D))
    q = rng.normal(size=(1, 1, D))
    wl = make_wl(keys, keys, q, [1], 16)
    _, sc = scores_of(wl)
    k = keys[0, 0, 0].astype(np.float32).astype(np.float64)
    exact = math.fsum(float(a) * float(c) for a, c in zip(q[0, 0].astype(np.float32), k))
    bound = (1 + math.log2(D)) * U * np.abs(q[0, 0].astype(np.float32) * k).sum() * 1.0001
    assert abs(sc[0, 0, 0] - exact) <= bound


@pytest.mark.parametrize("key,expect", [
    # D = 4, terms [1, 2^24, 1, -2^24]:
    #   balanced tree: fl(1 + 2^24) = 2^24 (tie to even); fl(1 - 2^24) = -(2^24 - 1);
    #                  sum = 1.  Left to right gives 0, pairing (0,2)(1,3) gives 2.
    ([1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)], 1.0),
    # D = 8, terms [2^24, 1, 1, 1, -2^24, 1, 1, 1]:
    #   level 1: 2^24, 2, -(2^24 - 1), 2;  level 2: 2^24 + 2, -(2^24 - 3);  total 5.
    #   Left to right gives 3, the exact sum is 6.
    ([2.0 ** 24, 1, 1, 1, -(2.0 ** 24), 1, 1, 1], 5.0),
])
def test_fixed_summation_order(key, expect):
    """The fp32 score is the balanced pairwise tree over contiguous channels."""
    D = len(key)
    keys = np.array(key, dtype=np.float32).reshape(1, 1, 1, D)
    q = np.ones((1, 1, D), dtype=np.float32)
    wl = make_wl(keys, keys, q, [1], 4)
    _, sc = scores_of(wl)
    assert sc[0, 0, 0] == np.float32(expect)


def test_score_doubles_with_query():
    wl = W.make("tinyllama", batch=2, context=700)
    meta, sc = scores_of(wl)
    sc2 = O.page_scores(wl.shape, wl.q * 2, meta, wl.block_table, wl.seq_lens)
    n = -(-700 // 16)
    assert np.array_equal(sc2[..., :n], sc[..., :n] * 2)


def test_integer_inputs_give_exact_scores():
    """Small-integer keys/queries: every product and sum exact; score = corner max."""
    wl = W.tie_heavy(11, head_dim=8, context=61, page_size=4, num_q_heads=6, num_kv_heads=2)
    sh = wl.shape
    G = sh.group
    meta, sc = scores_of(wl)
    for b in range(sh.batch):
        for h in range(sh.num_kv_heads):
            for p in range(-(-61 // 4)):
                phys = wl.block_table[b, p]
                mn = W.storage_to_f32(meta[phys, h, 0], sh.kv_dtype).astype(np.float64)
                mx = W.storage_to_f32(meta[phys, h, 1], sh.kv_dtype).astype(np.float64)
                exact = max(corner_max(wl.q[b, h * G + g], mn, mx) for g in range(G))
                assert sc[b, h, p] == exact


def one_token_pages(qs, key):
    """Score of a D = 1, one-token page whose key is `key` for G = len(qs)
    query heads (q_g = qs[g]), under both group aggregations."""
    G = len(qs)
    sh = W.Shape(1, G, 1, 1, 1, 1, 1, W.F32)
    kp = np.array([key], np.float32).reshape(1, 1, 1, 1)
    bt = np.zeros((1, 1), np.int32)
    lens = np.ones(1, np.int32)
    meta = O.meta_build(sh, kp, bt, lens)
    q = np.array(qs, np.float32).reshape(1, G, 1)
    return [float(O.page_scores(sh, q, meta, bt, lens, agg)[0, 0, 0])
            for agg in (O.AGG_MAX, O.AGG_SUM)]


def test_group_sum_fixed_order():
    """Sum over the group: fp32, heads in increasing order.  With per-head
    scores (1, 1e8, -1e8) that order gives (1 + 1e8) - 1e8 = 0 (1e8 + 1 rounds
    to 1e8), the reverse order 1, and the max 1e8."""
    assert one_token_pages([1.0, 1e8, -1e8], 1.0) == [1e8, 0.0]
    assert one_token_pages([-1e8, 1e8, 1.0], 1.0) == [1e8, 1.0]
    assert one_token_pages([3.0, -5.0], 2.0) == [6.0, -4.0]


def test_group_sum_is_sum_of_corner_maxima():
    """Small-integer inputs: the sum-aggregated score is exactly the sum over
    the group's heads of each head's box-corner maximum (brute force)."""
    rng = np.random.default_rng(17)
    D, G, P = 8, 4, 5
    keys = rng.integers(-3, 4, size=(1, 1, 3 * P, D)).astype(np.float32)
    q = rng.integers(-3, 4, size=(1, G, D)).astype(np.float32)
    wl = make_wl(keys, keys, q, [3 * P], P)
    sh = wl.shape
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    sc = O.page_scores(sh, wl.q, meta, wl.block_table, wl.seq_lens, O.AGG_SUM)
    for p in range(3):
        mn = meta[wl.block_table[0, p], 0, 0].astype(np.float64)
        mx = meta[wl.block_table[0, p], 0, 1].astype(np.float64)
        want = sum(corner_max(q[0, g], mn, mx) for g in range(G))
        assert sc[0, 0, p] == want


def test_group_sum_bounds_the_group_logit_sum():
    """Sum aggregation bounds sum_g q_g.k for every key of the page."""
    wl = W.make("tinyllama", batch=2, context=300)
    sh = wl.shape
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    sc = O.page_scores(sh, wl.q, meta, wl.block_table, wl.seq_lens, O.AGG_SUM)
    G, P = sh.group, sh.page_size
    for b in range(sh.batch):
        for h in range(sh.num_kv_heads):
            qs = wl.q[b, h * G:(h + 1) * G].astype(np.float64).sum(axis=0)
            for p in range(-(-300 // P)):
                k = page_pool_rows(wl, b, h, p)
                tight = (k @ qs).max()
                slack = 1e-5 * np.abs(wl.q[b, h * G:(h + 1) * G]).sum() * np.abs(k).max() * 2
                assert sc[b, h, p] >= tight - slack


# ----------------------------------------------------------------------------
# metadata
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [W.F32, W.F16, W.BF16, W.F8, W.F8E5])
def test_box_is_tightest(dtype):
    """Every valid key lies in the box and every face is attained by a valid key."""
    wl = W.make("gpt2", batch=3, context=77, kv_dtype=dtype)
    W.poison_unused(wl)
    sh = wl.shape
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    P = sh.page_size
    for b in range(sh.batch):
        for p in range(-(-77 // P)):
            for h in range(sh.num_kv_heads):
                k = page_pool_rows(wl, b, h, p)
                phys = wl.block_table[b, p]
                mn = W.storage_to_f32(meta[phys, h, 0], dtype).astype(np.float64)
                mx = W.storage_to_f32(meta[phys, h, 1], dtype).astype(np.float64)
                assert np.all(k >= mn) and np.all(k <= mx)
                assert np.all((k == mn).any(axis=0)) and np.all((k == mx).any(axis=0))


def test_append_matches_rebuild():
    """Appending token by token (including page opens) gives the rebuilt box."""
    wl = W.make("ragged", batch=4, lens_range=(20, 60), append_steps=19)
    sh = wl.shape
    pre = wl.steps[0].seq_lens - 1
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, pre)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    for st in wl.steps:
        O.meta_append(sh, st.k_new, st.v_new, kp, vp, meta, wl.block_table, st.seq_lens)
        rebuilt = O.meta_build(sh, kp, wl.block_table, st.seq_lens)
        P = sh.page_size
        for b in range(sh.batch):
            n = -(-int(st.seq_lens[b]) // P)
            phys = wl.block_table[b, :n]
            a = W.storage_to_f32(meta[phys], sh.kv_dtype)
            r = W.storage_to_f32(rebuilt[phys], sh.kv_dtype)
            assert np.array_equal(a, r)
        # the appended token sits in its slot
        for b in range(sh.batch):
            pos = int(st.seq_lens[b]) - 1
            phys = wl.block_table[b, pos // P]
            assert np.array_equal(kp[phys, :, pos % P], st.k_new[b])
            assert np.array_equal(vp[phys, :, pos % P], st.v_new[b])


# ----------------------------------------------------------------------------
# selection
# ----------------------------------------------------------------------------

def brute_force_selection(scores, n, K, n_sink, n_recent=0):
    """All subsets: the one whose members all beat all other candidates
    (sink pages first, then the most recent pages, are kept outright)."""
    keff = min(K, n)
    f = min(n_sink, keff)
    rec = min(n_recent, keff - f)
    cands = list(range(f, n - rec))
    r = keff - f - rec

    def beats(a, b):
        return scores[a] > scores[b] or (scores[a] == scores[b] and a < b)

    winners = []
    for sub in itertools.combinations(cands, r):
        s = set(sub)
        if all(beats(a, b) for a in s for b in cands if b not in s):
            winners.append(sorted(list(range(f)) + list(sub) + list(range(n - rec, n))))
    return winners


def test_selection_is_unique_dominant_subset():
    rng = np.random.default_rng(5)
    for trial in range(600):
        n = int(rng.integers(1, 10))
        K = int(rng.integers(1, 6))
        n_sink = int(rng.integers(0, min(K, 3) + 1))
        n_recent = int(rng.integers(0, K - n_sink + 1)) if trial % 2 else 0
        P = 2
        sh = W.Shape(1, 1, 1, 4, P, 10, 10, W.F32)
        scores = np.full((1, 1, 10), np.nan, dtype=np.float32)
        scores[0, 0, :n] = rng.integers(-2, 3, size=n).astype(np.float32)  # many ties
        lens = np.array([n * P - int(rng.integers(0, P))], dtype=np.int32)
        sel, cnt = O.select_from_scores(sh, scores, lens, K, None, n_sink, n_recent)
        winners = brute_force_selection(scores[0, 0], n, K, n_sink, n_recent)
        assert len(winners) == 1
        got = sel[0, 0, :cnt[0, 0]].tolist()
        assert got == winners[0]
        assert np.all(sel[0, 0, cnt[0, 0]:] == -1)


def test_selection_nesting_and_all_pages():
    wl = W.make("gpt2", batch=4, context=300)
    sh = wl.shape
    meta, sc = scores_of(wl)
    prev = None
    n = -(-300 // 16)
    for K in range(1, n + 3):
        sel, cnt = O.select_from_scores(sh, sc, wl.seq_lens, K)
        sets = [set(sel[b, h, :cnt[b, h]]) for b in range(sh.batch) for h in range(sh.num_kv_heads)]
        assert all(len(s) == min(K, n) for s in sets)
        if prev is not None:
            assert all(a <= c for a, c in zip(prev, sets))
        prev = sets
    assert all(s == set(range(n)) for s in prev)


def test_selection_independent_of_physical_layout():
    wl = W.make("tinyllama", batch=2, context=500)
    wl2 = W.make("tinyllama", batch=2, context=500, layout="permuted")
    # same logical content, different pool layout: rebuild wl2's pool from wl's
    sh = wl.shape
    for b in range(sh.batch):
        for p in range(sh.max_pages_per_seq):
            wl2.k_pool[wl2.block_table[b, p]] = wl.k_pool[wl.block_table[b, p]]
            wl2.v_pool[wl2.block_table[b, p]] = wl.v_pool[wl.block_table[b, p]]
    wl2.q = wl.q
    a = O.decode_step(sh, wl.q, wl.k_pool, wl.v_pool,
                      O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens),
                      wl.block_table, wl.seq_lens, 20, wl.scale)
    c = O.decode_step(sh, wl2.q, wl2.k_pool, wl2.v_pool,
                      O.meta_build(sh, wl2.k_pool, wl2.block_table, wl2.seq_lens),
                      wl2.block_table, wl2.seq_lens, 20, wl.scale)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
    assert np.array_equal(a[3], c[3])


def test_sink_page_always_kept():
    wl = W.make("llama_long", batch=2, context=2000)
    sh = wl.shape
    meta, sc = scores_of(wl)
    sel, cnt = O.select_from_scores(sh, sc, wl.seq_lens, wl.k_max, None, 1)
    assert np.all(sel[:, :, 0] == 0)
    assert np.all(cnt == min(wl.k_max, -(-2000 // 32)))


def test_recent_window_always_kept():
    """Sinks first, then the local window, then the best pages in between;
    K below sinks + window keeps the sinks and as much of the window as fits."""
    sh = W.Shape(1, 1, 1, 4, 1, 12, 12, W.F32)
    scores = np.array([[[5, 9, 1, 8, 2, 7, 3, 6, 0, 4, -1, -2]]], dtype=np.float32)
    lens = np.array([12], dtype=np.int32)

    def pick(K, n_sink, n_recent):   # row width 6, this row's budget K
        sel, cnt = O.select_from_scores(sh, scores, lens, 6, np.array([K], np.int32),
                                        n_sink, n_recent)
        return sel[0, 0, :cnt[0, 0]].tolist()

    assert pick(6, 1, 2) == [0, 1, 3, 5, 10, 11]   # sink 0, window 10-11, top-3 of 1..9
    assert pick(3, 1, 2) == [0, 10, 11]
    assert pick(2, 1, 2) == [0, 11]                # the budget cuts the window
    assert pick(4, 0, 4) == [8, 9, 10, 11]
    assert pick(5, 2, 3) == [0, 1, 9, 10, 11]
    with pytest.raises(RuntimeError):               # sinks + window beyond the row width
        O.select_from_scores(sh, scores, lens, 4, None, 2, 3)


def test_budget_clamped_and_zero_length():
    sh = W.Shape(3, 1, 1, 4, 2, 6, 18, W.F32)
    scores = np.arange(3 * 6, dtype=np.float32).reshape(3, 1, 6)
    lens = np.array([0, 5, 12], dtype=np.int32)
    sel, cnt = O.select_from_scores(sh, scores, lens, 4, np.array([9, 0, 2], np.int32), 0)
    assert cnt.tolist() == [[0], [1], [2]]          # len 0; K clamped to 1; K = 2
    assert sel[1, 0, 0] == 2 and sel[2, 0, :2].tolist() == [4, 5]


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def dense_attention_f64(wl):
    """Dense softmax attention over every valid token, float64, independent of the oracle."""
    sh = wl.shape
    G, P, D = sh.group, sh.page_size, sh.head_dim
    out = np.zeros((sh.batch, sh.num_q_heads, D))
    for b in range(sh.batch):
        L = int(wl.seq_lens[b])
        n = -(-L // P)
        k = W.storage_to_f32(wl.k_pool[wl.block_table[b, :n]], sh.kv_dtype).astype(np.float64)
        v = W.storage_to_f32(wl.v_pool[wl.block_table[b, :n]], sh.kv_dtype).astype(np.float64)
        k = k.transpose(1, 0, 2, 3).reshape(sh.num_kv_heads, n * P, D)[:, :L]
        v = v.transpose(1, 0, 2, 3).reshape(sh.num_kv_heads, n * P, D)[:, :L]
        for hq in range(sh.num_q_heads):
            z = float(wl.scale) * (k[hq // G] @ wl.q[b, hq].astype(np.float64))
            w = np.exp(z - z.max())
            out[b, hq] = (w / w.sum()) @ v[hq // G]
    return out


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict(context=333)),
    ("tinyllama", dict(batch=2, context=517)),
    ("ragged", dict(batch=3, lens_range=(30, 200), append_steps=0)),
    ("tinyllama", dict(batch=2, context=300, kv_dtype=W.F8)),
    ("gpt2", dict(batch=2, context=200, kv_dtype=W.F8E5)),
])
def test_all_pages_equals_dense_attention(name, kw):
    wl = W.make(name, **kw)
    W.poison_unused(wl)
    sh = wl.shape
    K = sh.max_pages_per_seq
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    _, _, _, out = O.decode_step(sh, wl.q, wl.k_pool, wl.v_pool, meta, wl.block_table,
                                 wl.seq_lens, K, wl.scale)
    ref = dense_attention_f64(wl)
    assert np.all(np.abs(out - ref) <= 1e-6 * np.maximum(1, np.abs(ref)))


def test_scale_zero_gives_mean_of_selected_values():
    wl = W.make("gpt2", batch=2, context=90)
    sh = wl.shape
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    sel, cnt, _ = O.select_pages(sh, wl.q, meta, wl.block_table, wl.seq_lens, 3)
    out = O.sparse_decode(sh, wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens,
                          sel, cnt, 3, 0.0)
    P = sh.page_size
    for b in range(sh.batch):
        for h in range(sh.num_q_heads):
            rows = []
            for p in sel[b, h, :cnt[b, h]]:
                v = min(P, 90 - p * P)
                rows.append(W.storage_to_f32(wl.v_pool[wl.block_table[b, p], h, :v], sh.kv_dtype))
            mean = np.concatenate(rows).astype(np.float64).mean(axis=0)
            assert np.allclose(out[b, h], mean, rtol=1e-6, atol=1e-7)


def test_constant_values_give_that_constant():
    """Every selected token carrying the same V row: out is that row, for any
    query and any selection (softmax weights sum to one)."""
    wl = W.make("ragged", batch=3, lens_range=(40, 400), append_steps=0)
    sh = wl.shape
    row = np.linspace(-2, 2, sh.head_dim).astype(np.float32)   # exact in fp16
    wl.v_pool[...] = W.to_storage(np.broadcast_to(row, wl.v_pool.shape), sh.kv_dtype)
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    _, cnt, _, out = O.decode_step(sh, wl.q, wl.k_pool, wl.v_pool, meta, wl.block_table,
                                   wl.seq_lens, wl.k_max, wl.scale, wl.k_per_seq)
    want = W.storage_to_f32(W.to_storage(row, sh.kv_dtype), sh.kv_dtype)
    assert np.all(cnt > 0)
    assert np.allclose(out, want[None, None, :], rtol=0, atol=1e-6)


def test_fma_form_of_the_term_is_bit_identical():
    """The per-channel term max(fl(q*mn), fl(q*mx)) equals the one-product
    form fl(q * (mx if q >= 0 else mn)) (the form a GPU evaluates as
    fma(min(q, 0), mn, max(q, 0) * mx)) on random triples with mn <= mx,
    signed zeros and wide exponents included; -0 compared as +0."""
    rng = np.random.default_rng(11)
    n = 200000
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    c = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    q = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    q[:100] = 0.0
    q[100:200] = -0.0
    a[200:300] = 0.0
    mn, mx = np.minimum(a, c), np.maximum(a, c)
    with np.errstate(over="ignore"):
        lhs = np.maximum(q * mn, q * mx)
        rhs = np.where(q >= 0, q * mx, q * mn)
    lhs[lhs == 0] = 0.0
    rhs[rhs == 0] = 0.0
    assert np.array_equal(lhs.view(np.uint32), rhs.view(np.uint32))


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    keys = rng.normal(size=(1, 1, 1, 64))
    vals = rng.normal(size=(1, 1, 1, 64))
    wl = make_wl(keys, vals, rng.normal(size=(1, 2, 64)), [1], 16)
    sh = wl.shape
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    _, cnt, _, out = O.decode_step(sh, wl.q, wl.k_pool, wl.v_pool, meta, wl.block_table,
                                   wl.seq_lens, 1, wl.scale)
    assert cnt.tolist() == [[1]]
    assert np.array_equal(out[0, 0], vals[0, 0, 0].astype(np.float32))
    assert np.array_equal(out[0, 1], vals[0, 0, 0].astype(np.float32))


def test_poisoned_slots_never_read():
    """NaN in every slot at or past the length leaves every result bit-identical."""
    wl = W.make("ragged", batch=4, lens_range=(17, 150), append_steps=0)
    sh = wl.shape
    clean = [wl.k_pool.copy(), wl.v_pool.copy()]
    W.poison_unused(wl)
    res = []
    for kp, vp in (clean, (wl.k_pool, wl.v_pool)):
        meta = O.meta_build(sh, kp, wl.block_table, wl.seq_lens)
        res.append(O.decode_step(sh, wl.q, kp, vp, meta, wl.block_table, wl.seq_lens,
                                 wl.k_max, wl.scale, wl.k_per_seq))
    for a, c in zip(res[0], res[1]):
        assert np.array_equal(a, c, equal_nan=True)
    assert np.all(np.isfinite(res[1][3]))


def test_empty_sequence_gives_zero_output():
    wl = W.make("tiny", batch=2, context=40)
    wl.seq_lens = np.array([0, 40], dtype=np.int32)
    sh = wl.shape
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    sel, cnt, _, out = O.decode_step(sh, wl.q, wl.k_pool, wl.v_pool, meta, wl.block_table,
                                     wl.seq_lens, 2, wl.scale)
    assert np.all(cnt[0] == 0) and np.all(sel[0] == -1)
    assert np.all(out[0] == 0) and np.all(cnt[1] == 2)
