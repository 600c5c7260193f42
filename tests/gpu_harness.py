"""Run the HIP path and the CPU oracle on the same seeded workload.

Shared by the GPU parity tests.  The HIP side goes through the C ABI (the
package binding); the oracle side through oracle/; both read the same input
arrays from workloads/.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle as O
import workloads as W

TOL = {W.F32: 1e-5, W.F16: 2e-3, W.BF16: 2e-3, W.F8: 2e-3, W.F8E5: 2e-3}
SYNC_BYTES = 2113536  # TSV_WORKSPACE_ZERO_BYTES: zero before and after every call


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_run(wl, k_max=None, k_per_seq="wl", n_sink=None, step=0, n_recent=0, group_agg=0):
    """Oracle results of one decode step (append first if the workload has steps)."""
    sh = wl.shape
    k_max = wl.k_max if k_max is None else k_max
    n_sink = wl.n_sink if n_sink is None else n_sink
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    if wl.steps:
        st = wl.steps[step]
        lens_pre = st.seq_lens - 1
        meta = O.meta_build(sh, kp, wl.block_table, lens_pre)
        kps = st.k_per_seq if isinstance(k_per_seq, str) else k_per_seq
        sel, cnt, sc, out = O.decode_step(sh, st.q, kp, vp, meta, wl.block_table, st.seq_lens,
                                          k_max, wl.scale, kps, n_sink, st.k_new, st.v_new,
                                          n_recent, group_agg)
    else:
        meta = O.meta_build(sh, kp, wl.block_table, wl.seq_lens)
        kps = wl.k_per_seq if isinstance(k_per_seq, str) else k_per_seq
        sel, cnt, sc, out = O.decode_step(sh, wl.q, kp, vp, meta, wl.block_table, wl.seq_lens,
                                          k_max, wl.scale, kps, n_sink, None, None,
                                          n_recent, group_agg)
    return dict(meta=meta, sel=sel, cnt=cnt, scores=sc, out=out, k_pool=kp, v_pool=vp)


def host_lengths(wl, k_max=None, k_per_seq="wl", step=0):
    """Host copies of the step's sequence lengths and budgets."""
    lens = wl.steps[step].seq_lens if wl.steps else wl.seq_lens
    if isinstance(k_per_seq, str):
        k_per_seq = wl.steps[step].k_per_seq if wl.steps else wl.k_per_seq
    return lens, k_per_seq


def lpt_order(wl, k_max=None, k_per_seq="wl", step=0, lib=None):
    """The library's longest-first row order for this step on this GPU."""
    import query_aware_sparse_bbox_amd as T_mod
    T = lib if lib is not None else T_mod
    k_max = wl.k_max if k_max is None else k_max
    cus, per = T.tsv_step_residency(wl.shape, k_max)
    lens, kps = host_lengths(wl, k_max, k_per_seq, step)
    return T.tsv_schedule_rows(wl.shape, k_max, lens, kps, cus, max(per, 1))


def gpu_run(wl, k_max=None, k_per_seq="wl", n_sink=None, step=0, separate=False, n_recent=0,
            group_agg=0, ws=None, lib=None, row_order=None):
    """HIP results of the same step; `separate` uses the three-call path.  With
    selection options the _ex entry points are called, else the plain ones.
    `ws`: a workspace to use (default: a new zero-filled one); the result's
    "sync" holds its counter prefix after the call.  `lib`: the library to call
    (default: the package's libtsv.so; the testing library for hooks).
    `row_order`: call tsv_decode_step_scheduled with this order (an int32
    array, or "lpt" for the library's own schedule)."""
    import torch

    import query_aware_sparse_bbox_amd as T_mod
    T = lib if lib is not None else T_mod
    from workloads import device as WD

    sh = wl.shape
    k_max = wl.k_max if k_max is None else k_max
    n_sink = wl.n_sink if n_sink is None else n_sink
    d = WD.upload(wl)
    B, Hq, Hkv, D, MP = sh.batch, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.max_pages_per_seq
    sel = torch.full((B, Hkv, k_max), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, Hkv, MP), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = T.new_workspace(sh, k_max)
    k_new = v_new = None
    if wl.steps:
        st = wl.steps[step]
        lens_pre = WD.i32(st.seq_lens - 1)
        T.tsv_meta_build(sh, d.k_pool, d.meta, d.block_table, lens_pre)
        seq_lens = WD.i32(st.seq_lens)
        q = torch.from_numpy(st.q).cuda()
        kps = WD.i32(st.k_per_seq) if isinstance(k_per_seq, str) else WD.i32(k_per_seq)
        k_new = WD.kv_tensor(st.k_new, sh.kv_dtype)
        v_new = WD.kv_tensor(st.v_new, sh.kv_dtype)
    else:
        seq_lens = d.seq_lens
        T.tsv_meta_build(sh, d.k_pool, d.meta, d.block_table, seq_lens)
        q = d.q
        kps = d.k_per_seq if isinstance(k_per_seq, str) else WD.i32(k_per_seq)
    if separate:
        if k_new is not None:
            T.tsv_meta_append(sh, k_new, v_new, d.k_pool, d.v_pool, d.meta, d.block_table,
                              seq_lens)
        if n_recent or group_agg:
            T.tsv_select_pages_ex(sh, q, d.meta, d.block_table, seq_lens, k_max, kps, n_sink,
                                  n_recent, group_agg, sel, cnt, sc, ws)
        else:
            T.tsv_select_pages(sh, q, d.meta, d.block_table, seq_lens, k_max, kps, n_sink,
                               sel, cnt, sc, ws)
        T.tsv_sparse_decode(sh, q, d.k_pool, d.v_pool, d.block_table, seq_lens, sel, cnt,
                            k_max, wl.scale, out, ws)
    elif row_order is not None:
        if isinstance(row_order, str):
            row_order = lpt_order(wl, k_max, k_per_seq, step, lib)
        ro = torch.from_numpy(np.ascontiguousarray(row_order, dtype=np.int32)).cuda()
        T.tsv_decode_step_scheduled(sh, q, k_new, v_new, d.k_pool, d.v_pool, d.meta,
                                    d.block_table, seq_lens, k_max, kps, n_sink, n_recent,
                                    group_agg, ro, wl.scale, sel, cnt, sc, out, ws)
    elif n_recent or group_agg:
        T.tsv_decode_step_ex(sh, q, k_new, v_new, d.k_pool, d.v_pool, d.meta, d.block_table,
                             seq_lens, k_max, kps, n_sink, n_recent, group_agg, wl.scale, sel,
                             cnt, sc, out, ws)
    else:
        T.tsv_decode_step(sh, q, k_new, v_new, d.k_pool, d.v_pool, d.meta, d.block_table,
                          seq_lens, k_max, kps, n_sink, wl.scale, sel, cnt, sc, out, ws)
    torch.cuda.synchronize()
    return dict(meta=WD.kv_numpy(d.meta, sh.kv_dtype), sel=sel.cpu().numpy(),
                cnt=cnt.cpu().numpy(), scores=sc.cpu().numpy(), out=out.cpu().numpy(),
                k_pool=WD.kv_numpy(d.k_pool, sh.kv_dtype), v_pool=WD.kv_numpy(d.v_pool, sh.kv_dtype),
                sync=ws[:SYNC_BYTES].cpu().numpy())


def n_pages(wl, step=0):
    lens = wl.steps[step].seq_lens if wl.steps else wl.seq_lens
    return (lens.astype(np.int64) + wl.shape.page_size - 1) // wl.shape.page_size


def compare(wl, g, o, step=0, check_meta=True):
    """Assert HIP results equal the oracle's: meta/scores/selection exact, out within tol."""
    sh = wl.shape
    n = n_pages(wl, step)
    if check_meta:
        for b in range(sh.batch):
            phys = wl.block_table[b, :n[b]]
            a = W.storage_to_f32(g["meta"][phys], sh.kv_dtype)
            r = W.storage_to_f32(o["meta"][phys], sh.kv_dtype)
            assert np.array_equal(a, r), f"meta differs in sequence {b}"
    for b in range(sh.batch):
        gs = g["scores"][b, :, :n[b]]
        os_ = o["scores"][b, :, :n[b]]
        if not np.array_equal(gs.view(np.uint32), os_.view(np.uint32)):
            bad = np.argwhere(gs.view(np.uint32) != os_.view(np.uint32))
            h, p = bad[0]
            raise AssertionError(f"score differs: b={b} h={h} p={p} gpu={gs[h, p]!r} "
                                 f"oracle={os_[h, p]!r} ({len(bad)} entries)")
    assert np.array_equal(g["cnt"], o["cnt"]), "sel_count differs"
    if not np.array_equal(g["sel"], o["sel"]):
        bad = np.argwhere(g["sel"] != o["sel"])
        raise AssertionError(f"selection differs at {bad[:5].tolist()} ({len(bad)} entries)")
    err = np.abs(g["out"].astype(np.float64) - o["out"].astype(np.float64))
    tol = TOL[sh.kv_dtype]
    assert np.all(np.isfinite(g["out"])), "non-finite output"
    assert err.max() <= tol, f"max-abs error {err.max():.3e} > {tol:.0e}"
    return float(err.max())
