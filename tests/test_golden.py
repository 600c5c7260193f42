"""Hand-derived golden cases (tests/golden/) against the oracle on the CPU and
against the HIP library on the GPU.

The expected values are written in the fixtures with their derivations from
the method's definition (TinyServe, "Query-Aware Cache Selection for
Efficient LLM Serving": method details, key design); neither implementation
produced them.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
D, P = 64, 16
AGG = {"max": O.AGG_MAX, "sum": O.AGG_SUM}


def cases(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)["cases"]


def _workload(q_rows, page_tokens, length):
    """One sequence, one KV head, fp32 KV: page p holds the rows page_tokens[p]."""
    G, n = len(q_rows), len(page_tokens)
    q = np.zeros((1, G, D), np.float32)
    for g, row in enumerate(q_rows):
        q[0, g, :len(row)] = row
    kp = np.zeros((n, 1, P, D), np.float32)
    for p, toks in enumerate(page_tokens):
        for t, row in enumerate(toks):
            kp[p, 0, t, :len(row)] = row
    sh = W.Shape(1, G, 1, D, P, n, n, W.F32)
    return W.Workload("golden", sh, kp, np.zeros_like(kp), q,
                      np.arange(n, dtype=np.int32).reshape(1, n),
                      np.array([length], np.int32), n, None, 0, 0.125)


def score_case(c):
    return _workload(c["q"], [c["tokens"]], len(c["tokens"]))


def selection_case(c):
    """Page p's valid tokens carry (scores[p], 0, ...) or rows[p]; slots past
    the length carry (junk, 0, ...)."""
    short, junk = c.get("short", 0), c.get("junk", 0)
    if "rows" in c:
        q_rows, rows = c["q"], c["rows"]
    else:
        q_rows, rows = [[1]], [[s] for s in c["scores"]]
    n = len(rows)
    length = n * P - short
    pages = []
    for p, row in enumerate(rows):
        valid = min(P, length - p * P)
        pages.append([row] * valid + [[junk]] * (P - valid))
    return _workload(q_rows, pages, length)


def _opts(c):
    kps = np.array([c["k_per_seq"]], np.int32) if "k_per_seq" in c else None
    return (c["k_max"], kps, c.get("n_sink", 0), c.get("n_recent", 0),
            AGG[c.get("group_agg", "max")])


# ---------------------------------------------------------------------------
# oracle (CPU)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("c", cases("score_cases.json"), ids=lambda c: c["name"])
def test_oracle_golden_scores(c):
    wl = score_case(c)
    sh = wl.shape
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    sc = O.page_scores(sh, wl.q, meta, wl.block_table, wl.seq_lens, AGG[c["group_agg"]])
    want = np.array(c["expect"], np.float32)
    assert np.array_equal(sc[0, 0, :len(want)].view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("c", cases("selection_cases.json"), ids=lambda c: c["name"])
def test_oracle_golden_selections(c):
    wl = selection_case(c)
    sh = wl.shape
    k_max, kps, n_sink, n_recent, agg = _opts(c)
    meta = O.meta_build(sh, wl.k_pool, wl.block_table, wl.seq_lens)
    sel, cnt, _ = O.select_pages(sh, wl.q, meta, wl.block_table, wl.seq_lens, k_max, kps,
                                 n_sink, n_recent, agg)
    assert sel[0, 0, :cnt[0, 0]].tolist() == c["expect"]
    assert np.all(sel[0, 0, cnt[0, 0]:] == -1)


# ---------------------------------------------------------------------------
# HIP library (GPU), through the C ABI
# ---------------------------------------------------------------------------

def _gpu_select(wl, k_max, kps, n_sink, n_recent, agg, fused):
    import torch

    import query_aware_sparse_bbox_amd as T
    from workloads import device as WD

    sh = wl.shape
    d = WD.upload(wl)
    T.tsv_meta_build(sh, d.k_pool, d.meta, d.block_table, d.seq_lens)
    sel = torch.full((1, 1, k_max), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1, 1), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((1, 1, sh.max_pages_per_seq), float("nan"), device="cuda")
    ws = T.new_workspace(sh, k_max)
    kp = WD.i32(kps)
    if fused:
        out = torch.empty((1, sh.num_q_heads, D), device="cuda")
        T.tsv_decode_step_ex(sh, d.q, None, None, d.k_pool, d.v_pool, d.meta, d.block_table,
                             d.seq_lens, k_max, kp, n_sink, n_recent, agg, wl.scale, sel, cnt,
                             sc, out, ws)
    else:
        T.tsv_select_pages_ex(sh, d.q, d.meta, d.block_table, d.seq_lens, k_max, kp, n_sink,
                              n_recent, agg, sel, cnt, sc, ws)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.gpu
@pytest.mark.parametrize("fused", [False, True], ids=["select", "step"])
@pytest.mark.parametrize("c", cases("score_cases.json"), ids=lambda c: c["name"])
def test_gpu_golden_scores(c, fused):
    wl = score_case(c)
    _, _, sc = _gpu_select(wl, 1, None, 0, 0, AGG[c["group_agg"]], fused)
    want = np.array(c["expect"], np.float32)
    assert np.array_equal(sc[0, 0, :len(want)].view(np.uint32), want.view(np.uint32))


@pytest.mark.gpu
@pytest.mark.parametrize("fused", [False, True], ids=["select", "step"])
@pytest.mark.parametrize("c", cases("selection_cases.json"), ids=lambda c: c["name"])
def test_gpu_golden_selections(c, fused):
    wl = selection_case(c)
    sel, cnt, _ = _gpu_select(wl, *_opts(c), fused)
    assert sel[0, 0, :cnt[0, 0]].tolist() == c["expect"]
    assert np.all(sel[0, 0, cnt[0, 0]:] == -1)
