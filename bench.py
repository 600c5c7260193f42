"""Benchmark one decode step of query-aware page selection + sparse paged decode.

A step is one tsv_decode_step_scheduled over one batch: [append one token per
sequence] -> score every page's box against the query -> keep the top-K pages
-> masked softmax attention over the kept pages only (TinyServe, "Query-Aware
Cache Selection for Efficient LLM Serving": abstract, method details), its
rows taken longest first in the order tsv_schedule_rows plans on the host from
the sequence lengths (planned once before the timed region, as a serving loop
plans a step from the lengths it keeps; the planning time is reported;
--schedule none: tsv_decode_step, rows in index order).  Inputs are
seeded synthetic tensors with the decode shapes of the pages' models,
resident in HBM before the timed region.  R copies of the pool and metadata
are rotated so that every step reads HBM rather than the 256 MB Infinity
Cache.  Steps are replayed from a HIP graph (--eager: launched one by one).

Prints one JSON line:
  value        (sequence x query head) / s of the whole step
  roofline     the step's algorithmic bytes / its mean duration (HIP events
               around the graph-replayed steps on their stream) against 8 TB/s;
               the step is one kernel (k_step; rows spread over several
               workgroups merge inside it); `traffic` = HBM bytes per
               step from rocprofv3 counters when they were taken on the current
               kernel source, else null
  cpu_baseline the CPU oracle, unchanged, on the same step: one sequence per
               task on a pool of host threads (median of 3 runs), plus a
               single-thread run; thread count and CPU model recorded
  selection_quality  share of the exact softmax mass (float64, sampled rows)
               that falls on the kept pages, and the same step with every page
               kept (dense) timed the same way

--copy-calibrate MB only runs a plain device copy of MB megabytes (the
reference kernel for scaling the HBM byte counters) and exits.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
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
DEFAULT_CONFIG = "ragged"
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
KERNEL_SOURCES = [os.path.join(ROOT, "query_aware_sparse_bbox_amd", "csrc", f)
                  for f in ("tsv_device.h", "tsv_kernels.hip", "tsv_host.hip", "tsv_api.hip",
                            "tsv_launch.h", "tsv_scratch.hip")]

# HBM bytes per step (all its kernels) from `rocprofv3 --pmc FETCH_SIZE` and
# `--pmc WRITE_SIZE` runs of this script, each divided by the same counter's
# reading per byte of a plain device copy (--copy-calibrate).  Valid only for
# the kernel source they were taken on (sha256 of KERNEL_SOURCES, first 16
# hex digits).  Keys: configuration, or configuration:KV type when the
# configuration's KV type is overridden.  Taken on the default launch (rows
# in the longest-first order); a row order moves the same bytes.
TRAFFIC = {
    "tinyllama": {"source": "27e82acaed2daea2", "bytes_per_step": 23270128, "read": 22223600, "written": 1046528},
    "tiny": {"source": "27e82acaed2daea2", "bytes_per_step": 587056, "read": 585776, "written": 1280},
    "gpt2": {"source": "27e82acaed2daea2", "bytes_per_step": 42706033, "read": 42525809, "written": 180224},
    "llama_long": {"source": "27e82acaed2daea2", "bytes_per_step": 202246762, "read": 202107498, "written": 139264},
    "ragged": {"source": "27e82acaed2daea2", "bytes_per_step": 403041398, "read": 401562626, "written": 1478772},
    "tinyllama:fp8e4m3": {"source": "27e82acaed2daea2", "bytes_per_step": 12844780, "read": 11798252, "written": 1046528},
    "llama_long:fp8e4m3": {"source": "27e82acaed2daea2", "bytes_per_step": 101714869, "read": 101575605, "written": 139264},
    "ragged:fp8e4m3": {"source": "27e82acaed2daea2", "bytes_per_step": 204396686, "read": 203058891, "written": 1337796},
}


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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
                total=meta + kv + qo + table + append)


def attention_mass_recall(keys, q, scale, page_size, kept_pages):
    """Share of each query head's exact softmax mass that falls on the kept
    pages, in float64.  keys [L][D]: the valid keys of one (sequence, KV head)
    in token order (token t on page t // page_size); q [G][D]: the group's
    queries; kept_pages: the kept logical pages.  Returns G floats."""
    keys = np.asarray(keys, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    L = keys.shape[0]
    page_of = np.arange(L) // page_size
    keep = np.zeros((L + page_size - 1) // page_size, dtype=bool)
    keep[np.asarray(list(kept_pages), dtype=np.int64)] = True
    out = []
    for g in range(q.shape[0]):
        z = (keys @ q[g]) * float(scale)
        w = np.exp(z - z.max())
        out.append(float(w[keep[page_of]].sum() / w.sum()))
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads(requested: int) -> int:
    """Threads for the oracle baseline: the CPUs this process may run on, at
    most 16 (the host share of one GPU), unless given explicitly."""
    if requested > 0:
        return requested
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(wl, st, lens_np, q_np, kps_np, k_max, n_sink, scale, args, agg):
    """The oracle's full step (append, score, select, attend) on the host."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle as O

    sh = wl.shape
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    meta = O.meta_build(sh, kp, wl.block_table, lens_np - 1 if st else lens_np)
    one = dataclasses.replace(sh, batch=1)
    kn = st.k_new if st else None
    vn = st.v_new if st else None

    def seq_step(b):
        O.decode_step(one, q_np[b:b + 1], kp, vp, meta, wl.block_table[b:b + 1],
                      lens_np[b:b + 1], k_max, scale,
                      None if kps_np is None else kps_np[b:b + 1], n_sink,
                      None if kn is None else kn[b:b + 1],
                      None if vn is None else vn[b:b + 1], args.recent, agg)

    def full_step(pool):
        if pool is None:
            for b in range(sh.batch):
                seq_step(b)
        else:
            list(pool.map(seq_step, range(sh.batch)))

    def timed(pool, min_s):
        reps, t = 0, 0.0
        while reps == 0 or t < min_s:
            c0 = time.perf_counter()
            full_step(pool)
            t += time.perf_counter() - c0
            reps += 1
        return t / reps, reps

    # single thread first (it also initialises the oracle's lookup tables)
    t1, reps1 = timed(None, args.cpu_seconds / 2)
    nthr = host_threads(args.cpu_threads)
    with ThreadPoolExecutor(max_workers=nthr) as pool:
        runs = [timed(pool, min(1.0, args.cpu_seconds / 6)) for _ in range(3)]
    tn = float(np.median([r[0] for r in runs]))
    B, Hq = sh.batch, sh.num_q_heads
    return {"value": B * Hq / tn, "unit": "(seq·head)/s", "cores": nthr, "kind": "oracle",
            "sample": f"the full decode step of the same workload (append, score, select, "
                      f"attend; boxes built beforehand), one sequence per task on {nthr} "
                      f"host threads, median of 3 runs of {runs[0][1]}+ step(s); single "
                      f"thread: {reps1} step(s)",
            "threads_step_ms": tn * 1e3,
            "runs_step_ms": [r[0] * 1e3 for r in runs],
            "single_thread_value": B * Hq / t1,
            "single_thread_step_ms": t1 * 1e3,
            "cpu_model": cpu_model(),
            "host_cpus_visible": os.cpu_count()}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=W.CONFIG_ORDER)
    ap.add_argument("--kv-dtype", default=None, choices=sorted(W.DTYPE_NAMES.values()),
                    help="store the KV cache in this type instead of the configuration's own")
    ap.add_argument("--group-agg", default="max", choices=["max", "sum"],
                    help="combine the G query heads' box bounds by max (default) or sum")
    ap.add_argument("--recent", type=int, default=0,
                    help="always keep the last N pages of every sequence (local window)")
    ap.add_argument("--rotate", type=int, default=0, help="pool copies (0: auto, >=512 MB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU-oracle baseline: minimum seconds of each single-thread "
                         "measurement (0 disables the leg)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads of the threaded oracle run (0: the CPUs this "
                         "process may use, at most 16)")
    ap.add_argument("--eager", action="store_true", help="launch steps one by one (no graph)")
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed steps for about this long before the warm-up steps, so that "
                         "the GPU's clocks have settled under this load (0: none)")
    ap.add_argument("--no-quality", action="store_true",
                    help="skip the selection-quality / dense-speedup report")
    ap.add_argument("--copy-calibrate", type=float, default=0.0, metavar="MB",
                    help="only run a plain device copy of MB megabytes, 5 times, and exit")
    ap.add_argument("--schedule", default="lpt", choices=["lpt", "none"],
                    help="row order of the step: the library's longest-first schedule "
                         "(default) or index order")
    ap.add_argument("--phases", action="store_true",
                    help="only print the one-launch step's per-workgroup phase times, from the "
                         "testing library's phase stamps over --steps eager steps, and exit")
    return ap.parse_args()


def copy_calibrate(mb):
    import torch
    n = int(mb * 1e6) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(5):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / 5
    print(json.dumps({"copy_bytes_each_way": n * 4, "ms": ms,
                      "gbs_read_plus_write": 2 * n * 4 / (ms * 1e-3) / 1e9}), flush=True)


PHASES = [("stage", 0, 1, "start -> block-table row staged (and the token appended)"),
          ("score", 1, 2, "page scoring, with a split row's key exchange"),
          ("select", 2, 3, "top-K selection"),
          ("decode", 3, 4, "attention over the kept pages' tokens"),
          ("finish", 4, 5, "combine of the waves' states, output (merge of split rows)")]


def plan_rows(T, sh, k_max, lens_np, kps_np, dev):
    """The library's longest-first row order for one step, on the device,
    and a record of it (with the host time the planning takes, median of 20)."""
    import torch

    import ctypes

    cus, per = T.tsv_step_residency(sh, k_max)
    times = []
    for _ in range(20):
        t = time.perf_counter()
        order = T.tsv_schedule_rows(sh, k_max, lens_np, kps_np, cus, max(per, 1))
        times.append(time.perf_counter() - t)
    # the C planner alone, on buffers set up once (what a serving loop in C
    # pays per step)
    shp = T.Shape.of(sh)
    lens32 = np.ascontiguousarray(lens_np, dtype=np.int32)
    kps32 = None if kps_np is None else np.ascontiguousarray(kps_np, dtype=np.int32)
    buf = np.empty(order.size, dtype=np.int32)
    n = ctypes.c_int32(0)
    args = (ctypes.byref(shp), int(k_max), ctypes.c_void_p(lens32.ctypes.data),
            None if kps32 is None else ctypes.c_void_p(kps32.ctypes.data), int(cus),
            int(max(per, 1)), ctypes.c_void_p(buf.ctypes.data), int(buf.size), ctypes.byref(n))
    c_times = []
    for _ in range(200):
        t = time.perf_counter()
        T._lib.tsv_schedule_rows(*args)
        c_times.append(time.perf_counter() - t)
    assert np.array_equal(buf, order)
    identity = order.size == sh.batch * sh.num_kv_heads and np.array_equal(
        order, np.arange(order.size))
    rec = {"kind": "lpt", "num_cus": cus, "per_cu": per, "used": per > 0 and not identity,
           "workgroups": int(order.size), "idle_workgroups": int((order < 0).sum()),
           "host_plan_us": float(np.median(c_times) * 1e6),
           "host_plan_us_via_python": float(np.median(times) * 1e6)}
    if identity:
        # rows of equal weight keep index order: the plain step does the same
        # without the order's load
        rec["identity"] = True
        return None, rec
    return torch.from_numpy(order).to(dev), rec


def phases(args, T, sh, wl, instance, q, k_new, v_new, bt, lens, k_max, kps, n_sink, scale,
           launches, order):
    """Phase times of the one-launch step from the testing library's stamps
    (100 MHz real-time counter, 10 ns ticks), per workgroup, over the last
    --steps eager steps (each read back right after its step)."""
    import torch

    if launches != 1:
        print(f"[phases] {args.config}: the step takes {launches} launches; phase stamps "
              "exist for the one-launch step only", flush=True)
        return
    t = T.testing_library()
    R = max(2, args.rotate or 2)
    insts = [instance() for _ in range(R)]
    torch.cuda.synchronize()

    def step(d):
        t.tsv_decode_step_scheduled(sh, q, k_new, v_new, d.k_pool, d.v_pool, d.meta, bt, lens,
                                    k_max, kps, n_sink, 0, 0, order, scale, d.sel, d.cnt, None,
                                    d.out, d.ws)

    for i in range(args.warmup):
        step(insts[i % R])
    torch.cuda.synchronize()
    per = {name: [] for name, *_ in PHASES}
    spans, totals = [], []
    for i in range(args.steps):
        step(insts[i % R])
        torch.cuda.synchronize()
        st = t.tsv_debug_phase_stamps(sh.kv_dtype).astype(np.int64)
        live = st[:, 5] > st[:, 0]
        live &= st[:, 0] > 0
        st = st[live]
        t0 = st[:, 0].min()
        spans.append((st[:, 5].max() - t0) / 100.0)
        totals.append(np.median(st[:, 5] - st[:, 0]) / 100.0)
        for name, a, b, _ in PHASES:
            per[name].append((st[:, b] - st[:, a]) / 100.0)
    cmd = "python3 bench.py " + " ".join(sys.argv[1:])
    lines = [f"# {args.config}" + (f" (KV {args.kv_dtype})" if args.kv_dtype else "") +
             ": one-launch step, phase times per workgroup" +
             (", rows in the longest-first order" if order is not None else ""), "",
             f"  {cmd}", "",
             f"  shape {sh}", f"  workgroups per step: {int(live.sum())}; "
             f"{args.steps} eager steps after {args.warmup} warm-up, each read back right after it",
             f"  kernel span (first start to last end) p50 {np.median(spans):.2f} us, "
             f"min {np.min(spans):.2f}, max {np.max(spans):.2f}",
             f"  workgroup life p50 {np.median(totals):.2f} us", "",
             f"  {'phase':<8}{'p10 us':>9}{'p50 us':>9}{'p90 us':>9}{'max us':>9}  what"]
    for name, a, b, what in PHASES:
        x = np.concatenate(per[name])
        lines.append(f"  {name:<8}{np.percentile(x, 10):>9.2f}{np.percentile(x, 50):>9.2f}"
                     f"{np.percentile(x, 90):>9.2f}{x.max():>9.2f}  {what}")
    print("\n".join(lines), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} / WORLD_SIZE {world} requested, but this library "
              "runs the decode step on one GPU only (no multi-GPU path); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.set_device(0)
    if args.copy_calibrate > 0:
        copy_calibrate(args.copy_calibrate)
        return

    import query_aware_sparse_bbox_amd as T
    from workloads import device as WD

    dev = "cuda"
    t_gen = time.time()
    dtype_of = {v: k for k, v in W.DTYPE_NAMES.items()}
    own_dtype = W.SPECS[args.config].kv_dtype
    kv_dtype = own_dtype if args.kv_dtype is None else dtype_of[args.kv_dtype]
    wl = W.make(args.config, kv_dtype=kv_dtype)
    sh = wl.shape
    st = wl.steps[0] if wl.steps else None
    lens_np = st.seq_lens if st else wl.seq_lens
    q_np = st.q if st else wl.q
    kps_np = st.k_per_seq if st else wl.k_per_seq
    print(f"[bench] {args.config}: {sh} generated in {time.time() - t_gen:.1f}s", flush=True)

    bt = WD.i32(wl.block_table)
    lens = WD.i32(lens_np)
    lens_pre = WD.i32(lens_np - 1) if st else lens
    q = torch.from_numpy(q_np).to(dev)
    kps = WD.i32(kps_np)
    k_new = WD.kv_tensor(st.k_new, sh.kv_dtype) if st else None
    v_new = WD.kv_tensor(st.v_new, sh.kv_dtype) if st else None
    k_max, n_sink, scale = wl.k_max, wl.n_sink, wl.scale
    B, Hq, Hkv, D = sh.batch, sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    launches = T.tsv_decode_step_launches(sh, k_max, st is not None)

    def instance():
        d = WD.upload(wl, dev)
        T.tsv_meta_build(sh, d.k_pool, d.meta, bt, lens_pre)
        d.sel = torch.empty((B, Hkv, k_max), dtype=torch.int32, device=dev)
        d.cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        d.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        d.ws = T.new_workspace(sh, k_max, dev)
        return d

    agg = {"max": T.TSV_AGG_MAX, "sum": T.TSV_AGG_SUM}[args.group_agg]
    variant = args.recent != 0 or agg != T.TSV_AGG_MAX
    order, sched = None, {"kind": "none"}
    if args.schedule == "lpt":
        order, sched = plan_rows(T, sh, k_max, lens_np, kps_np, dev)
        print(f"[bench] longest-first row order: {sched}", flush=True)

    def step(d):
        if order is not None:
            T.tsv_decode_step_scheduled(sh, q, k_new, v_new, d.k_pool, d.v_pool, d.meta, bt,
                                        lens, k_max, kps, n_sink, args.recent, agg, order,
                                        scale, d.sel, d.cnt, None, d.out, d.ws)
        elif variant:
            T.tsv_decode_step_ex(sh, q, k_new, v_new, d.k_pool, d.v_pool, d.meta, bt, lens,
                                 k_max, kps, n_sink, args.recent, agg, scale, d.sel, d.cnt,
                                 None, d.out, d.ws)
        else:
            T.tsv_decode_step(sh, q, k_new, v_new, d.k_pool, d.v_pool, d.meta, bt, lens, k_max,
                              kps, n_sink, scale, d.sel, d.cnt, None, d.out, d.ws)

    if args.phases:
        phases(args, T, sh, wl, instance, q, k_new, v_new, bt, lens, k_max, kps, n_sink, scale,
               launches, order)
        return

    first = instance()
    step(first)
    torch.cuda.synchronize()
    ref_sel, ref_out = first.sel.clone(), first.out.clone()
    nb = step_bytes(wl, lens_np, first.sel.cpu().numpy(), first.cnt.cpu().numpy())
    R = args.rotate or max(2, math.ceil(512e6 / nb["total"]))
    insts = [first] + [instance() for _ in range(R - 1)]
    torch.cuda.synchronize()
    print(f"[bench] {R} rotating instances, {nb['total'] / 1e6:.2f} MB algorithmic per step, "
          f"{launches} launch(es) per step", flush=True)

    stream = torch.cuda.current_stream()
    K, Wm = args.steps, args.warmup

    def capture(ds):
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            for d in ds:
                step(d)
        stream.wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for d in ds:
                step(d)
        torch.cuda.synchronize()
        return g

    graphs = {}

    def run(nsteps, marks=None):
        """Exactly nsteps steps, instance i % R for step i.  With `marks`, an
        event is recorded on the stream after every replay (every step when
        eager) and appended with the number of steps it closes."""
        def mark(count):
            if marks is not None:
                ev = torch.cuda.Event(enable_timing=True)
                ev.record(stream)
                marks.append((ev, count))

        if args.eager:
            for i in range(nsteps):
                step(insts[i % R])
                mark(1)
            return
        for _ in range(nsteps // R):
            graphs["full"].replay()
            mark(R)
        rem = nsteps % R
        if rem:
            if rem not in graphs:
                graphs[rem] = capture(insts[:rem])
            graphs[rem].replay()
            mark(rem)

    if not args.eager:
        graphs["full"] = capture(insts)
        for r in {K % R, Wm % R} - {0}:
            graphs[r] = capture(insts[:r])
        # a replayed step reproduces the eager one bit for bit
        first.sel.fill_(-5)
        first.out.fill_(float("nan"))
        graphs["full"].replay()
        torch.cuda.synchronize()
        assert torch.equal(first.sel, ref_sel), "graph replay changed the selection"
        assert torch.equal(first.out.view(torch.int32), ref_out.view(torch.int32)), \
            "graph replay changed the output"

    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle = 0
    if args.settle_ms > 0:
        t0.record(stream)
        run(R)
        t1.record(stream)
        torch.cuda.synchronize()
        settle = min(200000, max(R, math.ceil(args.settle_ms / max(t0.elapsed_time(t1) / R,
                                                                     1e-4))))
        run(settle)
        torch.cuda.synchronize()
    run(Wm)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    run(K)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / K
    # the median of per-replay step times, from a second pass of K steps with
    # an event after every replay (each closes R steps, or 1 when eager); the
    # events add small gaps, so the mean above is taken without them
    marks = []
    t0.record(stream)
    run(K, marks)
    torch.cuda.synchronize()
    per, prev = [], t0
    for ev, count in marks:
        per.append(prev.elapsed_time(ev) / count)
        prev = ev
    ms_median = float(np.median(per))
    print(f"[bench] step {ms_step * 1e3:.2f} us mean, {ms_median * 1e3:.2f} us median over "
          f"{len(per)} replays (wall {wall / K * 1e6:.2f} us/step)", flush=True)

    # selection quality: the share of exact softmax mass on the kept pages,
    # and the same step with every page kept (the dense baseline, same kernels)
    quality = None
    if not args.no_quality:
        MP = sh.max_pages_per_seq
        dense = []
        for d in insts:
            e = type("Dense", (), {})()
            e.sel = torch.empty((B, Hkv, MP), dtype=torch.int32, device=dev)
            e.cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
            e.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
            e.ws = T.new_workspace(sh, MP, dev)
            e.src = d
            dense.append(e)

        dorder = plan_rows(T, sh, MP, lens_np, None, dev)[0] if order is not None else None

        def dstep(e):
            d = e.src
            T.tsv_decode_step_scheduled(sh, q, k_new, v_new, d.k_pool, d.v_pool, d.meta, bt,
                                        lens, MP, None, n_sink, 0, 0, dorder, scale, e.sel,
                                        e.cnt, None, e.out, e.ws)

        s2 = torch.cuda.Stream()
        s2.wait_stream(stream)
        with torch.cuda.stream(s2):
            for e in dense:
                dstep(e)
        stream.wait_stream(s2)
        torch.cuda.synchronize()
        gd = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gd):
            for e in dense:
                dstep(e)
        reps = max(1, min(K, 100) // R)
        gd.replay()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(reps):
            gd.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms_dense = t0.elapsed_time(t1) / (reps * R)
        # recall on sampled (sequence, KV head) rows of the first instance,
        # in float64 from the pool after the step
        step(first)
        torch.cuda.synchronize()
        sel_np, cnt_np = first.sel.cpu().numpy(), first.cnt.cpu().numpy()
        P = sh.page_size
        units = B * Hkv
        rows = list(range(0, units, max(1, units // 32)))[:32]
        recalls = []
        for u in rows:
            b, h = divmod(u, Hkv)
            L = int(lens_np[b])
            n_pages = (L + P - 1) // P
            phys = torch.from_numpy(wl.block_table[b, :n_pages].astype(np.int64)).to(dev)
            kt = W.storage_to_f32(WD.kv_numpy(first.k_pool[phys, h].reshape(-1, D)[:L],
                                              sh.kv_dtype), sh.kv_dtype)
            recalls += attention_mass_recall(kt, q_np[b, h * sh.group:(h + 1) * sh.group],
                                             scale, P, sel_np[b, h, :cnt_np[b, h]])
        recalls = np.array(recalls)
        quality = {"attention_mass_recall_mean": float(recalls.mean()),
                   "attention_mass_recall_min": float(recalls.min()),
                   "rows_sampled": len(rows), "query_heads_sampled": int(recalls.size),
                   "dense_step_us": ms_dense * 1e3,
                   "sparse_speedup_vs_dense": ms_dense / ms_step,
                   "dense": "the same step with every page kept (k_max = max pages, its own "
                            "row order)"}
        print(f"[bench] dense step {ms_dense * 1e3:.2f} us, speedup {ms_dense / ms_step:.2f}x, "
              f"attention-mass recall mean {recalls.mean():.4f} min {recalls.min():.4f}",
              flush=True)
        del dense, gd

    # CPU oracle baseline on the same step: the oracle unchanged, one
    # sequence per task (its own block-table row, query, budget and appended
    # token; the pools are shared, each task writes only its own pages) on a
    # pool of host threads (ctypes releases the GIL), median of 3 runs; and a
    # single-thread run of the same tasks
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(wl, st, lens_np, q_np, kps_np, k_max, n_sink, scale, args, agg)
        print(f"[bench] cpu oracle {cpu['threads_step_ms']:.1f} ms/step on "
              f"{cpu['cores']} threads, {cpu['single_thread_step_ms']:.1f} ms/step on 1",
              flush=True)

    value = B * Hq / (ms_step * 1e-3)
    step_gbs = nb["total"] / (ms_step * 1e-3) / 1e9
    src = source_hash()
    tkey = args.config if kv_dtype == own_dtype else f"{args.config}:{W.DTYPE_NAMES[kv_dtype]}"
    tr = None if variant else TRAFFIC.get(tkey)
    traffic = tr["bytes_per_step"] if tr and tr["source"] == src else None
    kernel = {1: "k_step (append, score, select, decode of every row)"}.get(
        launches, f"tsv_decode_step phased path ({launches} kernels)")
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
        "config": {"workload": f"{args.config}: {DESCR[args.config]}" + (
                       "" if kv_dtype == own_dtype
                       else f" (KV stored as {W.DTYPE_NAMES[kv_dtype]} instead)"), "kv_dtype":
                   W.DTYPE_NAMES[sh.kv_dtype], "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "page_size": sh.page_size, "k_max": k_max,
                   "rotating_instances": R, "graph": not args.eager,
                   "untimed_settle_steps": settle, "row_schedule": sched,
                   "selection": {"n_sink": n_sink, "n_recent": args.recent,
                                 "group_agg": args.group_agg}},
        "step_algorithmic_bytes": nb["total"],
        "step_bytes_breakdown": {k: v for k, v in nb.items() if k != "total"},
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "achieved": step_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": step_gbs / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_step": nb["total"],
                     "launches_per_step": launches,
                     "mean_step_us": ms_step * 1e3,
                     "median_step_us": ms_median * 1e3,
                     "median_of": f"{len(per)} replays of {1 if args.eager else R} step(s), "
                                  "timed in a second pass with an event after each replay",
                     "timed_as": "HIP events on the launch stream around the graph-replayed "
                                 "steps, divided by the step count",
                     "kernel_source": src},
        "cpu_baseline": cpu,
        "selection_quality": quality,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
