"""Benchmark one decode step of query-aware page selection + sparse paged decode.

A step is one tsv_decode_step over one batch: [append one token per sequence]
-> score every page's box against the query -> keep the top-K pages -> masked
softmax attention over the kept pages only.  Inputs are seeded synthetic
tensors with the decode shapes of the pages' models (TinyServe, "Query-Aware
Cache Selection for Efficient LLM Serving"), resident in HBM before the timed
region.  R copies of the pool/metadata are rotated so that every step reads
HBM rather than the 256 MB Infinity Cache.

Prints one JSON line:
  value        (sequence x query head) / s of the whole step
  roofline     the split-decode kernel's algorithmic bytes / its mean duration
               (HIP events around each launch), against 8 TB/s
  cpu_baseline the CPU oracle (single thread) on a bounded sample of the step
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_HBM_GBS = 8000.0
METRIC = "sparse decode attention: (seq·head)/s + achieved HBM GB/s vs peak"
DEFAULT_CONFIG = "tinyllama"
DESCR = {
    "tiny": "tiny MHA decode: B=1, 4 heads, D=64, 1024 tokens, page 16, top-8, fp32 KV",
    "tinyllama": "TinyLLaMA-1.1B-shaped GQA decode: B=16, 32/4 heads, D=64, 4096 tokens, "
                 "page 16, 25% page budget (64 pages), bf16 KV",
    "gpt2": "GPT2-345M-shaped MHA decode: B=32, 16 heads, D=64, 1024 tokens, page 16, "
            "top-16, fp16 KV, permuted pool",
    "llama_long": "LLaMA-1.3B-shaped long-context decode: B=8, 32 heads, D=64, 32768 tokens, "
                  "page 32, 1/16 budget incl. 1 sink page, bf16 KV",
    "ragged": "ragged serving mix: B=64, 32/8 heads, D=128, lengths U[512,16384], page 16, "
              "budget min(64, 20%), fp16 KV, shared shuffled pool, 1 append per step",
}


# ---------------------------------------------------------------------------
# algorithmic bytes (what the method must move; implementation scratch excluded)
# ---------------------------------------------------------------------------

def step_bytes(wl, lens, sel, cnt):
    """Bytes per step: boxes of every page + valid K/V rows of selected pages +
    q in / out + block table [+ append: new K/V written, touched boxes r/w]."""
    sh = wl.shape
    e = W.DTYPE_BYTES[sh.kv_dtype]
    P, D = sh.page_size, sh.head_dim
    lens = lens.astype(np.int64)
    n = (lens + P - 1) // P
    meta = int(n.sum()) * sh.num_kv_heads * 2 * D * e
    kv = 0
    for b in range(sh.batch):
        for h in range(sh.num_kv_heads):
            pages = sel[b, h, :cnt[b, h]].astype(np.int64)
            v = np.minimum(P, lens[b] - pages * P)
            kv += int(v.sum()) * 2 * D * e
    qo = sh.batch * sh.num_q_heads * D * 4 * 2
    table = int(n.sum()) * 4
    append = sh.batch * sh.num_kv_heads * (2 * D * e + 2 * 2 * D * e) if wl.steps else 0
    return dict(meta=meta, kv=kv, q_out=qo, table=table, append=append,
                total=meta + kv + qo + table + append,
                decode_kernel=kv + sh.batch * sh.num_q_heads * D * 4)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=W.CONFIG_ORDER)
    ap.add_argument("--rotate", type=int, default=0, help="pool copies (0: auto, >=512 MB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU-oracle baseline budget (0 disables it)")
    ap.add_argument("--graph", action="store_true", help="replay the steps from a HIP graph")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} / WORLD_SIZE {world} requested, but this build "
              "runs the decode step on one GPU only (no multi-GPU path); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import query_aware_sparse_bbox_amd as T
    from workloads import device as WD

    torch.cuda.set_device(0)
    dev = "cuda"
    t_gen = time.time()
    wl = W.make(args.config)
    sh = wl.shape
    st = wl.steps[0] if wl.steps else None
    lens_np = st.seq_lens if st else wl.seq_lens
    q_np = st.q if st else wl.q
    kps_np = st.k_per_seq if st else wl.k_per_seq
    print(f"[bench] {args.config}: {sh} generated in {time.time() - t_gen:.1f}s", flush=True)

    # shared small inputs
    bt = WD.i32(wl.block_table)
    lens = WD.i32(lens_np)
    lens_pre = WD.i32(lens_np - 1) if st else lens
    q = torch.from_numpy(q_np).to(dev)
    kps = WD.i32(kps_np)
    k_new = WD.kv_tensor(st.k_new, sh.kv_dtype) if st else None
    v_new = WD.kv_tensor(st.v_new, sh.kv_dtype) if st else None
    k_max, n_sink, scale = wl.k_max, wl.n_sink, wl.scale
    B, Hq, Hkv, D, MP = sh.batch, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.max_pages_per_seq

    def instance():
        d = WD.upload(wl, dev)
        T.tsv_meta_build(sh, d.k_pool, d.meta, bt, lens_pre)
        d.sel = torch.empty((B, Hkv, k_max), dtype=torch.int32, device=dev)
        d.cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        d.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        d.ws = T.new_workspace(sh, k_max, dev)
        return d

    def step(d):
        T.tsv_decode_step(sh, q, k_new, v_new, d.k_pool, d.v_pool, d.meta, bt, lens, k_max,
                          kps, n_sink, scale, d.sel, d.cnt, None, d.out, d.ws)

    first = instance()
    step(first)
    torch.cuda.synchronize()
    nb = step_bytes(wl, lens_np, first.sel.cpu().numpy(), first.cnt.cpu().numpy())
    R = args.rotate or max(2, math.ceil(512e6 / nb["total"]))
    insts = [first] + [instance() for _ in range(R - 1)]
    torch.cuda.synchronize()
    print(f"[bench] {R} rotating instances, {nb['total'] / 1e6:.2f} MB algorithmic per step",
          flush=True)

    stream = torch.cuda.current_stream()
    K, Wm = args.steps, args.warmup
    graph = None
    if args.graph:
        # one graph holding R consecutive steps (one per instance)
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            for d in insts:
                step(d)
        stream.wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for d in insts:
                step(d)
        torch.cuda.synchronize()

    def run(nsteps):
        if graph is not None:
            for _ in range(nsteps // R):
                graph.replay()
            for i in range(nsteps % R):
                step(insts[i])
        else:
            for i in range(nsteps):
                step(insts[i % R])

    run(Wm)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    run(K)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / K
    print(f"[bench] step {ms_step * 1e3:.2f} us (wall {wall / K * 1e6:.2f} us/step)", flush=True)

    # dominant kernel: the split decode (+ its merge), timed per launch with events
    sel_cnt = [(d.sel, d.cnt) for d in insts]
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i in range(K):
        d = insts[i % R]
        ev[i][0].record(stream)
        T.tsv_sparse_decode(sh, q, d.k_pool, d.v_pool, bt, lens, d.sel, d.cnt, k_max, scale,
                            d.out, d.ws)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    dec_gbs = nb["decode_kernel"] / (dec_ms * 1e-3) / 1e9
    print(f"[bench] decode phase {dec_ms * 1e3:.2f} us/launch, {dec_gbs:.0f} GB/s", flush=True)
    del sel_cnt

    # CPU oracle baseline (single thread) on a bounded sample of the same step
    cpu = None
    if args.cpu_seconds > 0:
        import oracle as O
        kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
        meta = O.meta_build(sh, kp, wl.block_table, lens_np - 1 if st else lens_np)
        reps, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds:
            c0 = time.perf_counter()
            O.decode_step(sh, q_np, kp, vp, meta, wl.block_table, lens_np, k_max, scale,
                          kps_np, n_sink, st.k_new if st else None, st.v_new if st else None)
            t_cpu += time.perf_counter() - c0
            reps += 1
        cpu = {"value": B * Hq * reps / t_cpu, "unit": "(seq·head)/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{reps} full decode step(s) of the same workload "
                         f"({t_cpu:.1f} s, single-threaded C oracle, metadata prebuilt)"}
        print(f"[bench] cpu oracle {t_cpu / reps * 1e3:.1f} ms/step", flush=True)

    value = B * Hq / (ms_step * 1e-3)
    step_gbs = nb["total"] / (ms_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "(seq·head)/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {DESCR[args.config]}", "kv_dtype":
                   W.DTYPE_NAMES[sh.kv_dtype], "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "page_size": sh.page_size, "k_max": k_max,
                   "rotating_instances": R, "graph": bool(args.graph)},
        "step_algorithmic_bytes": nb["total"],
        "step_hbm_gbs": step_gbs,
        "step_frac_of_peak": step_gbs / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "kernel": "k_decode_split",
                     "achieved": dec_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": dec_gbs / PEAK_HBM_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": nb["decode_kernel"],
                     "mean_launch_us": dec_ms * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
