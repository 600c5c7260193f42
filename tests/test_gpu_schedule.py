"""The longest-first row schedule on the GPU (tsv_decode_step_scheduled).

The schedule decides only which workgroup runs which row and when, so the
scheduled step must give bitwise the plain step's results, which match the
oracle.  Covered: the ragged serving mix at full size in 16-bit and fp8 KV
with the library's own order (the launch the benchmark times), orders with
idle entries of every kind, more rows than resident workgroups (rows that
start as earlier workgroups finish), shapes that ignore the order (rows
spread over several workgroups; the phased path), and graph replay.
"""
import numpy as np
import pytest

import workloads as W
from gpu_harness import compare, gpu_run, lpt_order, oracle_run, say

pytestmark = pytest.mark.gpu


def assert_bitwise_equal(a, b):
    for k in ("sel", "cnt", "meta", "k_pool", "v_pool"):
        assert np.array_equal(a[k], b[k]), k
    for k in ("scores", "out"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


@pytest.mark.parametrize("dt", [W.F16, W.F8, W.F8E5])
def test_full_ragged_scheduled_matches_oracle(dt):
    wl = W.make("ragged", kv_dtype=dt)
    order = lpt_order(wl)
    say(f"[case] ragged {dt} order of {len(order)} ({int((order < 0).sum())} idle)")
    g = gpu_run(wl, row_order=order)
    o = oracle_run(wl)
    err = compare(wl, g, o)
    say(f"  max-abs err {err:.3e}")
    assert_bitwise_equal(g, gpu_run(wl))


def test_orders_with_idle_entries():
    wl = W.make("ragged", batch=40, lens_range=(16, 1500))  # 320 rows, one workgroup each
    U = wl.shape.batch * wl.shape.num_kv_heads
    plain = gpu_run(wl)
    compare(wl, plain, oracle_run(wl))
    rng = np.random.default_rng(7)
    for it in range(3):
        order = list(rng.permutation(U))
        for bad in (-1, -7, U, U + 5, 2**31 - 1, -(2**31)):
            order.insert(int(rng.integers(0, len(order) + 1)), bad)
        say(f"[case] permutation {it} with idle entries, {len(order)} workgroups")
        assert_bitwise_equal(gpu_run(wl, row_order=np.array(order, dtype=np.int64)), plain)
    say("[case] the library's order")
    assert_bitwise_equal(gpu_run(wl, row_order="lpt"), plain)


def test_more_rows_than_resident_workgroups():
    import query_aware_sparse_bbox_amd as T

    wl = W.make("ragged", batch=600, lens_range=(16, 800))  # 4800 rows
    cus, per = T.tsv_step_residency(wl.shape, wl.k_max)
    assert per >= 1
    order = lpt_order(wl)
    U = wl.shape.batch * wl.shape.num_kv_heads
    assert U > cus * per and len(order) == U  # a tail after the first wave
    say(f"[case] {U} rows on {cus} CUs x {per}")
    g = gpu_run(wl, row_order=order)
    compare(wl, g, oracle_run(wl))
    assert_bitwise_equal(g, gpu_run(wl))


def test_split_rows_ignore_the_order():
    import query_aware_sparse_bbox_amd as T

    wl = W.make("tinyllama", batch=4, context=2048)  # 16 rows, each over several workgroups
    assert T.tsv_step_residency(wl.shape, wl.k_max)[1] == 0
    U = wl.shape.batch * wl.shape.num_kv_heads
    plain = gpu_run(wl)
    assert_bitwise_equal(gpu_run(wl, row_order=np.arange(U)[::-1]), plain)
    assert_bitwise_equal(gpu_run(wl, row_order="lpt"), plain)


def test_phased_shape_ignores_the_order():
    import query_aware_sparse_bbox_amd as T

    wl = W.make("ragged", batch=2, lens_range=(65500, 65535), kv_dtype=W.BF16, num_q_heads=64)
    assert T.tsv_decode_step_launches(wl.shape, wl.k_max, True) > 1
    assert T.tsv_step_residency(wl.shape, wl.k_max)[1] == 0
    U = wl.shape.batch * wl.shape.num_kv_heads
    assert_bitwise_equal(gpu_run(wl, row_order=np.arange(U)[::-1]), gpu_run(wl))


def test_graph_replay_of_the_scheduled_step():
    """The scheduled step captured in a HIP graph and replayed, with eager
    work and synchronisations between replays, equals the eager step."""
    import torch

    import query_aware_sparse_bbox_amd as T
    from workloads import device as WD

    wl = W.make("ragged", batch=24, lens_range=(100, 3000))  # 192 rows
    sh = wl.shape
    st = wl.steps[0]
    d = WD.upload(wl)
    T.tsv_meta_build(sh, d.k_pool, d.meta, d.block_table, WD.i32(st.seq_lens - 1))
    B, Hq, Hkv, D = sh.batch, sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    order = torch.from_numpy(lpt_order(wl)).cuda()
    q = torch.from_numpy(st.q).cuda()
    lens, kps = WD.i32(st.seq_lens), WD.i32(st.k_per_seq)
    kn, vn = WD.kv_tensor(st.k_new, sh.kv_dtype), WD.kv_tensor(st.v_new, sh.kv_dtype)
    sel = torch.empty((B, Hkv, wl.k_max), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ws = T.new_workspace(sh, wl.k_max)

    def step():
        T.tsv_decode_step_scheduled(sh, q, kn, vn, d.k_pool, d.v_pool, d.meta, d.block_table,
                                    lens, wl.k_max, kps, 0, 0, 0, order, wl.scale, sel, cnt,
                                    None, out, ws)

    step()
    torch.cuda.synchronize()
    ref = (sel.clone(), cnt.clone(), out.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        sel.fill_(-5)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {i}")
        assert torch.equal(sel, ref[0]) and torch.equal(cnt, ref[1])
        assert torch.equal(out.view(torch.int32), ref[2].view(torch.int32))


@pytest.mark.parametrize("name,kw", [
    ("gpt2", dict(batch=40, context=700)),                                     # MHA, VALU decode
    ("gpt2", dict(batch=20, context=500, head_dim=128, kv_dtype=W.F32)),       # fp32 KV
    ("ragged", dict(batch=20, lens_range=(50, 1500), num_q_heads=128,          # G = 16
                    head_dim=64)),
    ("llama_long", dict(batch=6, context=3000, page_size=64, kv_dtype=W.F16)),  # 64-token pages
    ("ragged", dict(batch=24, lens_range=(20, 2500), kv_dtype=W.F8E5)),        # fp8, ragged
])
def test_scheduled_step_across_shapes(name, kw):
    """More than 128 rows, one workgroup each: the library's order and its
    reverse give the plain step's results bit for bit."""
    import query_aware_sparse_bbox_amd as T

    wl = W.make(name, **kw)
    U = wl.shape.batch * wl.shape.num_kv_heads
    assert U > 128 and T.tsv_step_residency(wl.shape, wl.k_max)[1] >= 1
    say(f"[case] {name} {kw}: {U} rows")
    plain = gpu_run(wl)
    order = lpt_order(wl)
    assert_bitwise_equal(gpu_run(wl, row_order=order), plain)
    assert_bitwise_equal(gpu_run(wl, row_order=order[::-1].copy()), plain)


@pytest.mark.parametrize("seed", range(6))
def test_scheduled_step_random_shapes(seed):
    """Seeded random one-launch shapes with more than 128 rows (group size,
    head dim, page size, KV type, ragged lengths, budget, sinks, appends):
    the library's order gives the plain step's results bit for bit."""
    import query_aware_sparse_bbox_amd as T

    rng = np.random.default_rng(500 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([2, 4, 8]))
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([8, 16, 32]))
    dt = [W.F16, W.BF16, W.F8, W.F8E5, W.F32][int(rng.integers(0, 5))]
    B = int(rng.integers(130 // Hkv + 1, 300 // Hkv + 1))
    hi = int(rng.integers(200, 3000))
    kw = dict(batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=P,
              kv_dtype=dt, lens_range=(1, hi), budget=("ragged", 32, 4),
              n_sink=int(rng.integers(0, 2)), append_steps=int(rng.integers(0, 2)))
    wl = W.make("ragged", **kw)
    say(f"[case] seed {seed}: {kw}")
    if T.tsv_step_residency(wl.shape, wl.k_max)[1] == 0:
        pytest.skip("shape takes the phased step")
    plain = gpu_run(wl)
    assert_bitwise_equal(gpu_run(wl, row_order="lpt"), plain)
