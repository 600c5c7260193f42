"""tsv_decode_step_noalloc (library-owned scratch, no workspace argument)
against tsv_decode_step_ex on the same inputs, through the C ABI.

Two calls in a row, the second with a smaller input, each compared with the
workspace entry point bit for bit (same kernels, same work split) and with
the oracle to the parity bar.  Both calls spread their rows over several
workgroups, so they go through the scratch's counter prefix, which each call
must leave at zero for the next.
"""
import numpy as np
import pytest

import workloads as W
from gpu_harness import compare, oracle_run, say

pytestmark = pytest.mark.gpu


def _run(wl, noalloc):
    import torch

    import query_aware_sparse_bbox_amd as T
    from workloads import device as WD

    sh = wl.shape
    st = wl.steps[0]
    d = WD.upload(wl)
    T.tsv_meta_build(sh, d.k_pool, d.meta, d.block_table, WD.i32(st.seq_lens - 1))
    B, Hq, Hkv, D, MP = sh.batch, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.max_pages_per_seq
    sel = torch.full((B, Hkv, wl.k_max), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, Hkv, MP), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    args = (sh, torch.from_numpy(st.q).cuda(), WD.kv_tensor(st.k_new, sh.kv_dtype),
            WD.kv_tensor(st.v_new, sh.kv_dtype), d.k_pool, d.v_pool, d.meta, d.block_table,
            WD.i32(st.seq_lens), wl.k_max, WD.i32(st.k_per_seq), wl.n_sink, 0, 0, wl.scale,
            sel, cnt, sc, out)
    if noalloc:
        T.tsv_decode_step_noalloc(*args)
    else:
        T.tsv_decode_step_ex(*args, T.new_workspace(sh, wl.k_max))
    torch.cuda.synchronize()
    return dict(meta=WD.kv_numpy(d.meta, sh.kv_dtype), sel=sel.cpu().numpy(),
                cnt=cnt.cpu().numpy(), scores=sc.cpu().numpy(), out=out.cpu().numpy(),
                k_pool=WD.kv_numpy(d.k_pool, sh.kv_dtype), v_pool=WD.kv_numpy(d.v_pool, sh.kv_dtype))


def test_noalloc_step_equals_workspace_step_twice():
    import query_aware_sparse_bbox_amd as T

    cases = [W.make("ragged", batch=6, lens_range=(300, 3000)),
             W.make("ragged", batch=3, lens_range=(40, 900), kv_dtype=W.BF16)]
    assert cases[1].shape.batch < cases[0].shape.batch
    for i, wl in enumerate(cases):
        need = T.tsv_workspace_bytes(wl.shape, wl.k_max)
        say(f"[case] noalloc call {i}: {wl.name} {wl.shape} workspace {need} B")
        assert 0 < need <= 33554432
        a = _run(wl, noalloc=True)
        b = _run(wl, noalloc=False)
        for k in ("sel", "cnt"):
            assert np.array_equal(a[k], b[k]), k
        for k in ("scores", "out"):
            assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
        for k in ("meta", "k_pool", "v_pool"):
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
        err = compare(wl, a, oracle_run(wl))
        say(f"  equal to the workspace step bit for bit; max-abs err vs oracle {err:.2e}")
