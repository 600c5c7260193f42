"""HIP path vs the CPU oracle, element by element, through the C ABI.

Bars: page boxes equal by value, page scores bit-equal (-0 stored as +0),
selections and counts bit-exact, outputs within max-abs 1e-5 (fp32 KV) or
2e-3 (fp16 / bf16 / fp8 KV: the stored values are exact in every path, the
tolerance covers the attention arithmetic).  The five decode configurations
run at their full sizes in the launch configuration the benchmark times;
smaller variants add ragged tails, several tiles per row and the method's
degenerate cases.
"""
import numpy as np
import pytest

import workloads as W
from gpu_harness import SYNC_BYTES, compare, gpu_run, oracle_run, say

pytestmark = pytest.mark.gpu


def _case(wl, **kw):
    say(f"[case] {wl.name} shape={wl.shape} kw={kw}")
    o = oracle_run(wl, **kw)
    say("  oracle done")
    g = gpu_run(wl, **kw)
    say("  gpu done")
    err = compare(wl, g, o, step=kw.get("step", 0))
    say(f"  max-abs err {err:.3e}")
    return g, o


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_full_config(name):
    wl = W.make(name)
    _case(wl)


@pytest.mark.parametrize("name,dt", [("tinyllama", W.F8), ("llama_long", W.F8),
                                     ("ragged", W.F8), ("tinyllama", W.F8E5),
                                     ("ragged", W.F8E5)])
def test_full_config_fp8(name, dt):
    """The same full-size steps with the KV cache stored as fp8 (E4M3, E5M2)."""
    wl = W.make(name, kv_dtype=dt)
    _case(wl)


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict(context=1000)),
    ("tiny", dict(context=17, kv_dtype=W.BF16)),
    ("tinyllama", dict(batch=3, context=1001)),
    ("tinyllama", dict(batch=2, context=333, num_q_heads=8, num_kv_heads=4)),  # G = 2
    ("gpt2", dict(batch=5, context=999)),
    ("gpt2", dict(batch=3, context=500, head_dim=128, kv_dtype=W.F32)),
    ("llama_long", dict(batch=2, context=5000)),
    ("llama_long", dict(batch=2, context=3000, page_size=64, kv_dtype=W.F16)),
    ("llama_long", dict(batch=2, context=3000, page_size=8)),
    ("ragged", dict(batch=8, lens_range=(1, 3000))),
    ("ragged", dict(batch=6, lens_range=(100, 2000), kv_dtype=W.BF16, num_q_heads=64)),
    # fp8 E4M3 KV: MFMA decode (G = 8, 4), VALU decode (G = 1, 2), 8-token pages
    ("tinyllama", dict(batch=3, context=1001, kv_dtype=W.F8)),
    ("tinyllama", dict(batch=2, context=333, num_q_heads=8, num_kv_heads=4, kv_dtype=W.F8)),
    ("tinyllama", dict(batch=2, context=777, page_size=8, kv_dtype=W.F8)),
    ("gpt2", dict(batch=3, context=500, kv_dtype=W.F8)),
    ("gpt2", dict(batch=2, context=700, head_dim=128, kv_dtype=W.F8)),
    ("ragged", dict(batch=6, lens_range=(100, 2000), kv_dtype=W.F8)),
    ("ragged", dict(batch=4, lens_range=(1, 1500), kv_dtype=W.F8, num_q_heads=64)),
    # fp8 E5M2 KV: MFMA decode (G = 8, 4), VALU decode (G = 1), 8-token pages
    ("tinyllama", dict(batch=3, context=1001, kv_dtype=W.F8E5)),
    ("tinyllama", dict(batch=2, context=777, page_size=8, kv_dtype=W.F8E5)),
    ("gpt2", dict(batch=3, context=500, kv_dtype=W.F8E5)),
    ("ragged", dict(batch=6, lens_range=(100, 2000), kv_dtype=W.F8E5)),
    ("llama_long", dict(batch=2, context=3000, kv_dtype=W.F8E5)),
])
def test_small_variants(name, kw):
    wl = W.make(name, **kw)
    _case(wl)


@pytest.mark.parametrize("dtype", [W.F32, W.F16, W.BF16, W.F8, W.F8E5])
@pytest.mark.parametrize("G", [1, 4])
def test_tie_heavy(dtype, G):
    wl = W.tie_heavy(31 + G, kv_dtype=dtype, num_q_heads=2 * G, num_kv_heads=2, context=777,
                     k_max=9, n_sink=1, value_range=2)
    g, o = _case(wl)
    # ties must actually occur among the scores for the case to mean anything
    sc = o["scores"][:, :, :49]
    assert max(len(v) - len(set(v.tolist())) for v in sc.reshape(-1, 49)) > 5


# selection variants: group sum aggregation (MFMA and VALU decode, both
# paths), a forced recent window with and without sinks, budgets that cut the
# window, tie-heavy rows
@pytest.mark.parametrize("name,kw,opts", [
    ("tinyllama", dict(batch=3, context=1001), dict(group_agg=1)),
    ("tinyllama", dict(batch=2, context=333, num_q_heads=8, num_kv_heads=4), dict(group_agg=1)),
    ("ragged", dict(batch=6, lens_range=(100, 2000)), dict(group_agg=1, n_recent=3)),
    ("llama_long", dict(batch=2, context=5000), dict(n_recent=4)),
    ("llama_long", dict(batch=2, context=3000, kv_dtype=W.F8), dict(n_recent=2, group_agg=1)),
    ("gpt2", dict(batch=5, context=999), dict(n_recent=1, n_sink=1)),
    ("ragged", dict(batch=8, lens_range=(1, 600)), dict(n_recent=2, n_sink=1, k_max=4)),
])
def test_selection_variants(name, kw, opts):
    wl = W.make(name, **kw)
    o = dict(opts)
    if "k_max" in o:
        o["k_per_seq"] = None
    _case(wl, **o)


def test_selection_variants_phased_and_full_size():
    import query_aware_sparse_bbox_amd as T

    wl = W.make("tinyllama")
    _case(wl, group_agg=1, n_recent=2)
    # the phased path (three calls) and a 4095-page row (phased one-call step)
    wl = W.make("ragged", batch=4, lens_range=(100, 3000))
    o = oracle_run(wl, group_agg=1, n_recent=2)
    g = gpu_run(wl, group_agg=1, n_recent=2, separate=True)
    compare(wl, g, o)
    wl = W.make("ragged", batch=2, lens_range=(65500, 65535), kv_dtype=W.BF16, num_q_heads=64)
    assert T.tsv_decode_step_launches(wl.shape, wl.k_max, True) == 4
    _case(wl, group_agg=1, n_recent=5)


@pytest.mark.parametrize("G", [1, 4])
def test_selection_variants_tie_heavy(G):
    wl = W.tie_heavy(41 + G, kv_dtype=W.BF16, num_q_heads=2 * G, num_kv_heads=2, context=777,
                     k_max=9, n_sink=1, value_range=2)
    _case(wl, group_agg=1, n_recent=2)


def test_poisoned_unused_slots():
    for name, kw in [("gpt2", dict(batch=4, context=301)),
                     ("ragged", dict(batch=8, lens_range=(5, 900))),
                     ("tinyllama", dict(batch=3, context=333, kv_dtype=W.F8)),
                     ("gpt2", dict(batch=3, context=250, kv_dtype=W.F8)),
                     ("tinyllama", dict(batch=3, context=333, kv_dtype=W.F8E5))]:
        wl = W.make(name, **kw)
        W.poison_unused(wl)
        g, _ = _case(wl)
        assert np.all(np.isfinite(g["out"]))


def test_all_pages_is_dense_attention():
    wl = W.make("tinyllama", batch=2, context=1500)
    _case(wl, k_max=wl.shape.max_pages_per_seq)
    wl = W.make("ragged", batch=4, lens_range=(50, 1200), append_steps=0)
    _case(wl, k_max=wl.shape.max_pages_per_seq, k_per_seq=None)


# Accepted shapes that the configurations above do not reach, each on the
# one-launch step and on the three-call (phased) path: the MFMA decode with
# 32- and 64-token pages (groups of 4 and 8, 16-bit and fp8 KV) and with
# 8-token pages on fp16, fp32 KV with groups of 2, 8 and 16, and groups of 16
# query heads (scoring in two head slices, decode in passes) in every KV type,
# with the maximum and the sum over the group.
SWEEP = [
    ("tinyllama", dict(batch=2, context=1500, page_size=32, kv_dtype=W.BF16), {}),
    ("tinyllama", dict(batch=2, context=3000, page_size=64, kv_dtype=W.F16), {}),
    ("tinyllama", dict(batch=2, context=1500, page_size=32, kv_dtype=W.F8), {}),
    ("tinyllama", dict(batch=2, context=3000, page_size=64, kv_dtype=W.F8E5), {}),
    ("ragged", dict(batch=3, lens_range=(100, 2000), page_size=32), {}),
    ("ragged", dict(batch=3, lens_range=(100, 3000), page_size=64, kv_dtype=W.BF16), {}),
    ("ragged", dict(batch=3, lens_range=(100, 1500), page_size=32, kv_dtype=W.F8), {}),
    ("tinyllama", dict(batch=2, context=700, page_size=8, kv_dtype=W.F16), {}),
    ("tinyllama", dict(batch=2, context=900, num_q_heads=8, num_kv_heads=4, kv_dtype=W.F32), {}),
    ("tinyllama", dict(batch=2, context=900, kv_dtype=W.F32), {}),
    ("tinyllama", dict(batch=2, context=900, head_dim=128, kv_dtype=W.F32), {}),
    ("tinyllama", dict(batch=2, context=1200, num_q_heads=64, num_kv_heads=4), {}),
    ("tinyllama", dict(batch=2, context=1200, num_q_heads=64, num_kv_heads=4),
     dict(group_agg=1)),
    ("tinyllama", dict(batch=2, context=1200, num_q_heads=32, num_kv_heads=2, head_dim=128,
                       kv_dtype=W.F16), {}),
    ("tinyllama", dict(batch=2, context=800, num_q_heads=32, num_kv_heads=2, kv_dtype=W.F32),
     {}),
    ("tinyllama", dict(batch=2, context=800, num_q_heads=32, num_kv_heads=2, head_dim=128,
                       kv_dtype=W.F32), dict(group_agg=1)),
    ("tinyllama", dict(batch=2, context=1000, num_q_heads=64, num_kv_heads=4, kv_dtype=W.F8),
     {}),
    ("tinyllama", dict(batch=2, context=1000, num_q_heads=64, num_kv_heads=4,
                       kv_dtype=W.F8E5, page_size=32), dict(group_agg=1, n_recent=2)),
    ("ragged", dict(batch=2, lens_range=(50, 1500), num_q_heads=128), {}),
    ("ragged", dict(batch=2, lens_range=(50, 1500), num_q_heads=128, kv_dtype=W.F32),
     dict(group_agg=1)),
    # VALU decode on fp8 (G = 1 and 2): tiles of twice the tokens of 16-bit KV
    ("llama_long", dict(batch=2, context=4096, kv_dtype=W.F8), {}),
    ("ragged", dict(batch=3, lens_range=(100, 3000), num_q_heads=16, kv_dtype=W.F8E5), {}),
]


@pytest.mark.parametrize("name,kw,opts", SWEEP,
                         ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(SWEEP)])
def test_shape_sweep(name, kw, opts):
    wl = W.make(name, **kw)
    o = oracle_run(wl, **opts)
    compare(wl, gpu_run(wl, **opts), o)
    compare(wl, gpu_run(wl, separate=True, **opts), o)
    say(f"  {name} {kw} {opts}: one-launch and phased paths match")


def test_scores_with_wide_single_wave_selection():
    """The select overwrites the page keys in local memory with the kept
    page indices, so the exported scores are copied out before it: with more
    than 64 pages kept (300-page rows, budget 128, the workgroup select) they
    must still be the page scores, on the one-launch step and the three-call
    path."""
    wl = W.make("tinyllama", batch=2, context=300 * 16 - 5)
    assert wl.shape.max_pages_per_seq >= 300
    g, o = _case(wl, k_max=128, k_per_seq=None)
    assert o["cnt"].min() == 128
    g = gpu_run(wl, k_max=128, k_per_seq=None, separate=True)
    compare(wl, g, o)


def test_three_calls_equal_fused_step():
    """tsv_meta_append + tsv_select_pages + tsv_sparse_decode give the same
    selection, boxes and pools as tsv_decode_step; both outputs are within
    tolerance of the oracle (their summation orders differ)."""
    import query_aware_sparse_bbox_amd as T

    for name, kw in [("ragged", dict(batch=8, lens_range=(100, 4000))),
                     ("tinyllama", dict(batch=4, context=2000)),
                     ("llama_long", dict(batch=2, context=6000)),
                     ("ragged", dict(batch=4, lens_range=(100, 3000), kv_dtype=W.F8)),
                     ("gpt2", dict(batch=4, context=600, kv_dtype=W.F8))]:
        wl = W.make(name, **kw)
        say(f"[case] three calls vs one step: {name} {kw} launches="
            f"{T.tsv_decode_step_launches(wl.shape, wl.k_max, bool(wl.steps))}")
        o = oracle_run(wl)
        a = gpu_run(wl)
        b = gpu_run(wl, separate=True)
        for k in ("sel", "cnt", "meta", "k_pool", "v_pool", "scores"):
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
        compare(wl, a, o)
        compare(wl, b, o)


def test_one_launch_and_phased_paths_both_covered():
    """The five configurations take the one-launch step; 4096-entry block
    table rows with a group of eight 128-channel heads take the phased path
    (row staging plus the group's combine area exceed 64 KiB)."""
    import query_aware_sparse_bbox_amd as T

    for name in W.CONFIG_ORDER:
        wl = W.make(name)
        # one launch each (tinyllama's 64 rows are each spread over several
        # workgroups that merge in the same kernel)
        assert T.tsv_decode_step_launches(wl.shape, wl.k_max, bool(wl.steps)) == 1, name
    wl = W.make("ragged", batch=2, lens_range=(65500, 65535), kv_dtype=W.BF16, num_q_heads=64)
    assert wl.shape.max_pages_per_seq >= 4064
    assert T.tsv_decode_step_launches(wl.shape, wl.k_max, True) == 4
    _case(wl)


def test_longest_block_table_row():
    """4096 pages per row: the largest row the library accepts, every thread
    of the selection owning several pages."""
    wl = W.make("llama_long", batch=1, num_q_heads=4, num_kv_heads=4, context=131072)
    assert wl.shape.max_pages_per_seq == 4096
    _case(wl)
    wl = W.make("llama_long", batch=1, num_q_heads=2, num_kv_heads=2, context=131072 - 77,
                budget=("fixed", 200))
    _case(wl)


def test_graph_replay_matches_eager():
    """The step captured in a HIP graph and replayed several times, with eager
    work and synchronisations between replays, equals the eager step."""
    import torch

    import query_aware_sparse_bbox_amd as T
    from workloads import device as WD

    wl = W.make("ragged", batch=8, lens_range=(100, 3000))
    sh = wl.shape
    st = wl.steps[0]
    d = WD.upload(wl)
    T.tsv_meta_build(sh, d.k_pool, d.meta, d.block_table, WD.i32(st.seq_lens - 1))
    B, Hq, Hkv, D = sh.batch, sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    args = dict(q=torch.from_numpy(st.q).cuda(), k_new=WD.kv_tensor(st.k_new, sh.kv_dtype),
                v_new=WD.kv_tensor(st.v_new, sh.kv_dtype), lens=WD.i32(st.seq_lens),
                kps=WD.i32(st.k_per_seq))
    sel = torch.empty((B, Hkv, wl.k_max), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ws = T.new_workspace(sh, wl.k_max)

    def step():
        T.tsv_decode_step(sh, args["q"], args["k_new"], args["v_new"], d.k_pool, d.v_pool,
                          d.meta, d.block_table, args["lens"], wl.k_max, args["kps"], 0,
                          wl.scale, sel, cnt, None, out, ws)

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


def test_multi_layer_graph_with_per_layer_budgets():
    """Four layers of a decode step, each with its own pools, KV type, budget
    and selection options, captured in one HIP graph: every eager layer
    matches the oracle, every replay (eager work and synchronisations
    between replays) reproduces the eager results bit for bit."""
    import torch

    import query_aware_sparse_bbox_amd as T
    from workloads import device as WD

    specs = [  # (KV type, k_max, per-sequence budgets?, n_sink, n_recent, group_agg)
        (W.BF16, 24, True, 0, 0, 0),
        (W.BF16, 16, False, 0, 0, 1),
        (W.F8, 32, True, 1, 2, 0),
        (W.F16, 8, False, 1, 1, 1),
    ]
    layers = []
    for i, (dt, k_max, per_seq, n_sink, n_recent, agg) in enumerate(specs):
        wl = W.make("tinyllama", seed=500 + i, batch=4, context=1500, kv_dtype=dt)
        sh = wl.shape
        kps = wl.k_per_seq if per_seq else None
        if kps is not None:
            kps = np.minimum(kps, k_max).astype(np.int32)
        o = oracle_run(wl, k_max=k_max, k_per_seq=kps, n_sink=n_sink, n_recent=n_recent,
                       group_agg=agg)
        d = WD.upload(wl)
        T.tsv_meta_build(sh, d.k_pool, d.meta, d.block_table, d.seq_lens)
        B, Hq, Hkv, D = sh.batch, sh.num_q_heads, sh.num_kv_heads, sh.head_dim
        L = dict(wl=wl, sh=sh, d=d, o=o, k_max=k_max, kps=WD.i32(kps), n_sink=n_sink,
                 n_recent=n_recent, agg=agg,
                 sel=torch.empty((B, Hkv, k_max), dtype=torch.int32, device="cuda"),
                 cnt=torch.empty((B, Hkv), dtype=torch.int32, device="cuda"),
                 sc=torch.empty((B, Hkv, sh.max_pages_per_seq), device="cuda"),
                 out=torch.empty((B, Hq, D), device="cuda"), ws=T.new_workspace(sh, k_max))
        layers.append(L)

    def step():
        for L in layers:
            d = L["d"]
            T.tsv_decode_step_ex(L["sh"], d.q, None, None, d.k_pool, d.v_pool, d.meta,
                                 d.block_table, d.seq_lens, L["k_max"], L["kps"], L["n_sink"],
                                 L["n_recent"], L["agg"], L["wl"].scale, L["sel"], L["cnt"],
                                 L["sc"], L["out"], L["ws"])

    def results():
        return [(L["sel"].cpu().numpy(), L["cnt"].cpu().numpy(), L["sc"].cpu().numpy(),
                 L["out"].cpu().numpy()) for L in layers]

    step()
    torch.cuda.synchronize()
    eager = results()
    for i, (L, (sel, cnt, sc, out)) in enumerate(zip(layers, eager)):
        g = dict(meta=WD.kv_numpy(L["d"].meta, L["sh"].kv_dtype), sel=sel, cnt=cnt, scores=sc,
                 out=out)
        err = compare(L["wl"], g, L["o"])
        say(f"  layer {i}: k_max {L['k_max']}, max-abs err {err:.2e}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        for L in layers:
            L["sel"].fill_(-5)
            L["out"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (a_sel, a_cnt, a_sc, a_out), (b_sel, b_cnt, b_sc, b_out) in zip(eager, results()):
            assert np.array_equal(a_sel, b_sel) and np.array_equal(a_cnt, b_cnt)
            assert np.array_equal(a_out.view(np.uint32), b_out.view(np.uint32))
        say(f"  replay {r} equals eager")


def test_bitwise_deterministic():
    wl = W.make("tinyllama", batch=4, context=2048)
    a, b = gpu_run(wl), gpu_run(wl)
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
    assert np.array_equal(a["scores"].view(np.uint32), b["scores"].view(np.uint32))


def test_split_count_does_not_change_result():
    """A wider sel row (more split slots) with the same budgets gives identical bits."""
    wl = W.make("llama_long", batch=2, context=4000)
    kp = np.full(wl.shape.batch, wl.k_max, dtype=np.int32)
    a = gpu_run(wl, k_max=wl.k_max, k_per_seq=kp)
    b = gpu_run(wl, k_max=wl.k_max + 40, k_per_seq=kp)
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
    assert np.array_equal(a["sel"], b["sel"][:, :, :wl.k_max])


def test_degenerate_lengths_and_budgets():
    wl = W.make("tinyllama", batch=5, context=300)
    wl.seq_lens = np.array([0, 1, 16, 17, 300], dtype=np.int32)
    g, o = _case(wl, k_max=3, k_per_seq=np.array([9, 0, 1, 2, 3], np.int32), n_sink=1)
    assert g["cnt"][0].tolist() == [0, 0, 0, 0] and np.all(g["out"][0] == 0)
    _case(wl, k_max=2, k_per_seq=None, n_sink=2)   # every slot forced
    _case(wl, k_max=40, k_per_seq=None, n_sink=0)  # K > n for every row


def test_permuted_pool_same_selection():
    a = W.make("tinyllama", batch=3, context=900)
    b = W.make("tinyllama", batch=3, context=900, layout="permuted")
    for bb in range(a.shape.batch):
        for p in range(a.shape.max_pages_per_seq):
            b.k_pool[b.block_table[bb, p]] = a.k_pool[a.block_table[bb, p]]
            b.v_pool[b.block_table[bb, p]] = a.v_pool[a.block_table[bb, p]]
    b.q = a.q
    ga, gb = gpu_run(a), gpu_run(b)
    assert np.array_equal(ga["sel"], gb["sel"])
    assert np.array_equal(ga["out"].view(np.uint32), gb["out"].view(np.uint32))


@pytest.mark.parametrize("kw", [dict(batch=16), dict(batch=8, kv_dtype=W.F8),
                                dict(batch=4), dict(batch=2, kv_dtype=W.F8E5)])
def test_ragged_appends_seventeen_steps(kw):
    """17 consecutive appends cover every slot residue mod 16 and page opens.
    With 4 and 2 sequences every row is spread over several workgroups, each
    of which appends the token before reading any box or slot."""
    import torch

    import oracle as O
    import query_aware_sparse_bbox_amd as T
    from workloads import device as WD

    wl = W.make("ragged", append_steps=17, **kw)
    sh = wl.shape
    say(f"[case] ragged appends shape={sh}")
    d = WD.upload(wl)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    lens0 = wl.steps[0].seq_lens - 1
    meta_o = O.meta_build(sh, kp, wl.block_table, lens0)
    T.tsv_meta_build(sh, d.k_pool, d.meta, d.block_table, WD.i32(lens0))
    B, Hq, Hkv, D = sh.batch, sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    sel = torch.empty((B, Hkv, wl.k_max), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hkv, sh.max_pages_per_seq), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ws = T.new_workspace(sh, wl.k_max)
    for i, st in enumerate(wl.steps):
        so, co, sco, oo = O.decode_step(sh, st.q, kp, vp, meta_o, wl.block_table, st.seq_lens,
                                        wl.k_max, wl.scale, st.k_per_seq, 0, st.k_new, st.v_new)
        T.tsv_decode_step(sh, torch.from_numpy(st.q).cuda(), WD.kv_tensor(st.k_new, sh.kv_dtype),
                          WD.kv_tensor(st.v_new, sh.kv_dtype), d.k_pool, d.v_pool, d.meta,
                          d.block_table, WD.i32(st.seq_lens), wl.k_max, WD.i32(st.k_per_seq), 0,
                          wl.scale, sel, cnt, sc, out, ws)
        torch.cuda.synchronize()
        g = dict(meta=WD.kv_numpy(d.meta, sh.kv_dtype), sel=sel.cpu().numpy(),
                 cnt=cnt.cpu().numpy(), scores=sc.cpu().numpy(), out=out.cpu().numpy())
        o = dict(meta=meta_o, sel=so, cnt=co, scores=sco, out=oo)
        err = compare(wl, g, o, step=i)
        say(f"  step {i}: max-abs err {err:.3e}")
    # the incrementally kept boxes equal a rebuild from the pool
    rebuilt = torch.zeros_like(d.meta)
    T.tsv_meta_build(sh, d.k_pool, rebuilt, d.block_table, WD.i32(wl.steps[-1].seq_lens))
    torch.cuda.synchronize()
    n = (wl.steps[-1].seq_lens + 15) // 16
    a, r = WD.kv_numpy(d.meta, sh.kv_dtype), WD.kv_numpy(rebuilt, sh.kv_dtype)
    for b in range(B):
        phys = wl.block_table[b, :n[b]]
        assert np.array_equal(W.storage_to_f32(a[phys], sh.kv_dtype),
                              W.storage_to_f32(r[phys], sh.kv_dtype))
    assert np.array_equal(WD.kv_numpy(d.k_pool, sh.kv_dtype), kp)
    assert np.array_equal(WD.kv_numpy(d.v_pool, sh.kv_dtype), vp)
    assert not ws[:SYNC_BYTES].cpu().numpy().any(), "split-row counters left non-zero"


def test_split_rows_exchange_fallback_bit_identical():
    """Rows spread over several workgroups share their page scoring through the
    workspace.  With the wait cut to zero polls (testing library), every split
    scores the rest of its row itself: scores, selections and outputs are the
    same bits, and the counters and key slots are left at zero either way."""
    import query_aware_sparse_bbox_amd as T

    t = T.testing_library()
    wl = W.make("tinyllama", batch=4, context=4096)
    assert T.tsv_decode_step_launches(wl.shape, wl.k_max, False) == 1
    o = oracle_run(wl)
    a = gpu_run(wl)
    compare(wl, a, o)
    prev = t.tsv_debug_exchange_polls(0)
    try:
        b = gpu_run(wl, lib=t)
        wl8 = W.make("tinyllama", batch=2, context=4096, kv_dtype=W.F8)
        compare(wl8, gpu_run(wl8, lib=t), oracle_run(wl8))
    finally:
        t.tsv_debug_exchange_polls(prev)
    for k in ("sel", "cnt"):
        assert np.array_equal(a[k], b[k]), k
    for k in ("scores", "out"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    assert not a["sync"].any() and not b["sync"].any()


@pytest.mark.parametrize("name,kw", [("tinyllama", dict(batch=4, context=4096)),
                                     ("gpt2", dict(batch=12, context=900))])
def test_phase_stamps_of_the_testing_library(name, kw):
    """The testing library's step kernels stamp every workgroup's phases: for
    each workgroup of the last step the stamps are non-decreasing from start
    to end, the recorded (row, split) pairs cover every row's splits once,
    and the results equal the library proper's bit for bit."""
    import query_aware_sparse_bbox_amd as T

    t = T.testing_library()
    wl = W.make(name, **kw)
    sh = wl.shape
    say(f"[case] phase stamps {name} {kw}")
    a = gpu_run(wl)
    b = gpu_run(wl, lib=t)
    st = t.tsv_debug_phase_stamps(sh.kv_dtype).astype(np.int64)
    for k in ("sel", "cnt"):
        assert np.array_equal(a[k], b[k]), k
    for k in ("scores", "out"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    units = sh.batch * sh.num_kv_heads
    S = T.tsv_decode_step_launches(sh, wl.k_max, bool(wl.steps))  # 1: one launch
    assert S == 1
    ids = st[:, 6]
    rows, splits = ids >> 32, ids & 0xffffffff
    # workgroups of this launch: stamped within 1 ms of its latest start (the
    # array keeps earlier launches' stamps in rows this grid does not reach)
    live = ((st[:, 5] >= st[:, 0]) & (st[:, 0] >= st[:, 0].max() - 100_000) &
            (rows < units))
    st, rows, splits = st[live], rows[live], splits[live]
    pairs = set(zip(rows.tolist(), splits.tolist()))
    assert len(pairs) == len(rows), "a (row, split) stamped twice"
    assert set(rows.tolist()) == set(range(units))
    nsplit = max(splits) + 1
    assert len(rows) == units * nsplit
    # start <= staged <= scored <= selected <= decoded <= end (decoded is only
    # stamped by workgroups that had tokens)
    for i0, i1 in ((0, 1), (1, 2), (2, 3), (3, 5)):
        assert (st[:, i1] >= st[:, i0]).all(), (i0, i1)
    span_us = (st[:, 5].max() - st[:, 0].min()) / 100.0
    assert 0 < span_us < 10000, span_us


def test_split_rows_workspace_shared_by_shapes():
    """One zero-filled workspace serves split-row steps of different shapes (and
    a phased call in between); each call leaves the counter prefix at zero."""
    import query_aware_sparse_bbox_amd as T

    a = W.make("tinyllama", batch=4, context=4096)
    b = W.make("ragged", batch=3, lens_range=(200, 3000), append_steps=1)
    n = max(T.tsv_workspace_bytes(a.shape, a.k_max), T.tsv_workspace_bytes(b.shape, b.k_max))
    import torch
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for wl, kw in ((a, {}), (b, {}), (a, dict(separate=True)), (b, {}), (a, {})):
        say(f"[case] shared workspace: {wl.name} {wl.shape} {kw}")
        g = gpu_run(wl, ws=ws, **kw)
        compare(wl, g, oracle_run(wl))
        assert not g["sync"].any()
