#!/usr/bin/env python3
"""Benchmark of the TT-EmbeddingBag hot path on one MI355X.

Workload: one 11,000,000-row table (radices 200x220x250), dim 128 (4x8x4),
TT rank 32, fp32 cores; a batch of 32,768 bags with Poisson(20) lengths
clipped to [1,100] and unpermuted Zipf(1.1) indices; grad_out ~ N(0,1) and an
SGD step with lr 0.01. One step is the whole path on one batch: plan (split,
prefix grouping, chunking, row runs), forward (the training call, which keeps
each group's prefix product for the backward), then the backward fused with
the SGD step (the cores updated in place on the slices the batch touches;
bit for bit the separate backward and SGD calls, whose times are reported
too), with every input already resident in HBM.

Steps run as a training loop would run them: the plan of the next batch needs
only that batch's indices, so it is built on a second stream, into a second
workspace, while the current batch's forward and backward run; each forward
still waits for the previous step's SGD update, and each plan for the step
that last used its workspace. `ms_per_step` is that loop's time per step;
`ms_per_step_serial` times the same steps one after another on one stream.

Prints one JSON line: whole-step pooled bags/s as `value`; per-call times of
each phase (HIP events around back-to-back calls on the stream the kernels run
on); the forward call's roofline figures; and the CPU oracle timed on a
bounded sample of the same batch as `cpu_baseline`.

Rooflines: every kernel's average duration comes from HIP events the
library records around each launch on the stream it launches on
(tt_emb_set_timing), in an instrumented pass after the timed region. The work
counted is the work the kernels execute: the forward contracts each distinct
table row of a prefix group once, so k_fwd_batch does U * 2*n1*n2*R^2
(prefixes) + U_row * 2*n1*n2*n3*R (suffixes of distinct rows) FLOP, k_pool
L * D adds; the per-lookup count of the plain method is reported beside it
as context. `roofline` is k_fwd_batch (the forward's dominant kernel);
`roofline_forward_call` adds pooling; `roofline_step` lists every kernel of
the training step with its fp32 and fp64 FLOP (fractions of 157.3 and 78.6
TFLOP/s) or its algorithmic bytes (each datum counted once, a fraction of
8 TB/s; the gather kernels also give their rate of per-lookup row reads,
most of which hit L2 or the Infinity Cache). HBM traffic comes
from rocprofv3 counter passes kept under profiles/ and is reported only while
the kernel sources still match the hash recorded there.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3      # MI355X published dense FP32 (matrix cores and vector)
PEAK_HBM_GBS = 8000.0         # MI355X published HBM3E bandwidth
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kernel_traffic_skew11m.json")
CSRC = os.path.join(ROOT, "tensor_train_compressed_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--chunk", type=int, default=256)
    ap.add_argument("--cpu-bags", type=int, default=32768,
                    help="bags of the batch the CPU oracle baseline runs on (0: skip)")
    ap.add_argument("--phase-reps", type=int, default=50)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of 256 MiB (reference for HBM counters)")
    ap.add_argument("--hot-rows", type=int, default=0,
                    help="instead of the main line: the training step with a hot-row cache of the batch's "
                         "N most frequent rows, beside the same step without it (one JSON line)")
    ap.add_argument("--forward-workload", default=None, choices=["tiny", "table1m", "skew11m", "multi26"],
                    help="instead of the training step: plan and forward of this workload only "
                         "(one JSON line with its forward rooflines)")
    return ap.parse_args()


def forward_only(args):
    """Plan and forward of one workload (tiny: 1,000 rows, rank 4; table1m:
    1M rows, rank 16, 4,096 bags; skew11m: the training workload's table and
    batch; multi26: 26 tables of 10^3 to 4*10^7 rows, dim 64 = 4x4x4, rank
    32, 32,768 bags per table, 8.5 M lookups): per-call times and the forward
    kernels' rooflines, as for the main workload."""
    import numpy as np
    import torch

    import tensor_train_compressed_amd as tte
    import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    p = wl.make(args.forward_workload)
    t0 = p.tables[0]
    n1, n2, n3 = t0.n
    R, D = t0.rank, t0.dim
    T, B, L = p.T, p.batch, p.L
    tabs = tte.make_tables(p.tables, p.goff)
    g = [torch.from_numpy(x).to(dev) for x in (p.g1, p.g2, p.g3)]
    idx = torch.from_numpy(p.indices).to(dev)
    off = torch.from_numpy(p.offsets).to(dev)
    out = torch.empty((T * B, D), dtype=torch.float32, device=dev)
    ws = torch.empty(tte.tt_emb_workspace_bytes(tabs, L, B, args.chunk), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    plan = lambda: tte.tt_emb_plan(tabs, idx, off, B, args.chunk, workspace=ws, stream=stream)
    pl = plan()
    q = tte.tt_emb_query_paths(pl, g[0], g[1])
    for _ in range(args.warmup):
        pl = plan()
        tte.tt_emb_forward(pl, g[0], g[1], g[2], out, stream=stream)
    torch.cuda.synchronize()
    assert tte.tt_emb_get_error(pl) == 0

    def per_call_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = args.steps
    plan_ms = per_call_ms(plan, reps)
    pl = plan()
    fwd_ms = per_call_ms(lambda: tte.tt_emb_forward(pl, g[0], g[1], g[2], out, stream=stream), reps)
    tte.tt_emb_set_timing(pl, True)
    for _ in range(reps):
        tte.tt_emb_forward(pl, g[0], g[1], g[2], out, stream=stream)
    recs = tte.tt_emb_kernel_times(pl, stream)
    tte.tt_emb_set_timing(pl, False)
    agg = {}
    for k, ms in recs:
        agg.setdefault(k, []).append(ms)
    us = {k: 1e3 * sum(v) / len(v) for k, v in agg.items()}
    # executed work: one prefix product per (table, i1, i2) group, one suffix
    # product per distinct (table, row), one add per lookup
    bag = np.repeat(np.arange(T * B), np.diff(p.offsets))
    tab = bag // B
    m3 = np.array([t.m[2] for t in p.tables], dtype=np.int64)[tab]
    U = int(np.unique(tab * (1 << 40) + p.indices // m3).size)
    U_row = int(np.unique(tab * (1 << 40) + p.indices).size)
    pre = U * 2 * n1 * n2 * R * R
    suf = U_row * 2 * n1 * n2 * n3 * R
    # the matrix-core kernels, or the generic one (which pools as it goes)
    kname = "k_fwd_batch" if "k_fwd_batch" in us else "k_fwd_generic"
    kb, kp = us.get(kname, 0.0) * 1e-6, us.get("k_pool", 0.0) * 1e-6
    fwd_bytes = 8 * L + 8 * (T * B + 1) + 4 * (p.g1.size + p.g2.size + p.g3.size) + 4 * T * B * D
    res = {
        "metric": f"pooled bags/s, TT-EmbeddingBag forward of the {args.forward_workload} batch",
        "value": round(T * B / (fwd_ms * 1e-3), 1), "unit": "bags/s", "n_gpus": 1, "higher_is_better": True,
        "dtype": "f32", "data": "synthetic (seeded Zipf/Poisson indices, Gaussian cores)",
        "config": {"workload": f"{args.forward_workload}: {T} tables, dim {D}={n1}x{n2}x{n3}, rank {R}, "
                               f"B={B} bags per table", "lookups": L, "prefix_groups": U, "distinct_rows": U_row},
        "paths": {"forward": q["forward_path"], "workspace_bytes": q["workspace_bytes"]},
        "phases_ms_per_call": {"plan": round(plan_ms, 4), "forward": round(fwd_ms, 4)},
        "kernels_us": {k: round(v, 2) for k, v in sorted(us.items(), key=lambda x: -x[1])},
        "roofline": {"kernel": kname, "bound": "mfma" if kname == "k_fwd_batch" else "alu",
                     "achieved": round((pre + suf) / kb / 1e12, 3),
                     "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round((pre + suf) / kb / 1e12 / PEAK_FP32_TFLOPS, 4), "flop_per_launch": int(pre + suf)},
        "roofline_forward_call": {"kernels": f"{kname} + k_pool" if kp > 0 else kname, "us": round((kb + kp) * 1e6, 2),
                                  "flop": int(pre + suf + L * D),
                                  "frac": round((pre + suf + L * D) / (kb + kp) / 1e12 / PEAK_FP32_TFLOPS, 4)
                                  if kb + kp > 0 else None},
        "plan_forward_bags_per_s": round(T * B / ((plan_ms + fwd_ms) * 1e-3), 1),
        "forward_rows_per_s": round(L / (fwd_ms * 1e-3), 1),
        # indices, offsets, cores once, pooled rows out
        "forward_algorithmic_bytes": int(fwd_bytes),
        "forward_hbm_gbs_algorithmic": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 1),
    }
    print(json.dumps(res))


def hot_rows_step(args):
    """The training step (plan, training forward, backward fused with SGD)
    on the main workload with a hot-row cache of the batch's N most frequent
    rows (uncompressed, trainable, started at their TT values), against the
    same step without the cache, both one step after another on one
    stream."""
    import numpy as np
    import torch

    import tensor_train_compressed_amd as tte
    import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    p = wl.make("train11m")
    B, L, D = p.batch, p.L, p.tables[0].dim
    tabs = tte.make_tables(p.tables, p.goff)
    g = [torch.from_numpy(x).to(dev) for x in (p.g1, p.g2, p.g3)]
    idx = torch.from_numpy(p.indices).to(dev)
    off = torch.from_numpy(p.offsets).to(dev)
    gout = torch.from_numpy(p.grad_out).to(dev)
    out = torch.empty((B, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    rows, cnt = np.unique(p.indices, return_counts=True)
    top = rows[np.argsort(-cnt, kind="stable")[:args.hot_rows]]
    n_hot = int(top.size)
    served = float(cnt[np.argsort(-cnt, kind="stable")[:args.hot_rows]].sum()) / L
    cache = tte.HotCache(torch.zeros(n_hot, dtype=torch.int32, device=dev), torch.from_numpy(top).to(dev))
    # W starts at the rows' TT values: a plain forward of one-lookup bags
    hot_w = torch.empty((n_hot, D), dtype=torch.float32, device=dev)
    tp = tte.tt_emb_plan(tabs, torch.from_numpy(top).to(dev),
                         torch.arange(n_hot + 1, dtype=torch.int64, device=dev), n_hot, args.chunk)
    tte.tt_emb_forward(tp, g[0], g[1], g[2], hot_w)
    ws = torch.empty(tte.tt_emb_workspace_bytes(tabs, L, B, args.chunk), dtype=torch.uint8, device=dev)

    def step_cached():
        pl = tte.tt_emb_plan(tabs, idx, off, B, args.chunk, workspace=ws, stream=stream, cache=cache)
        tok = tte.tt_emb_forward_cached(pl, g[0], g[1], g[2], hot_w, out, keep=True, stream=stream)
        tte.tt_emb_backward_sgd_cached(pl, tok, g[0], g[1], g[2], hot_w, gout, p.lr, stream=stream)
        return pl

    def step_plain():
        pl = tte.tt_emb_plan(tabs, idx, off, B, args.chunk, workspace=ws, stream=stream)
        tok = tte.tt_emb_forward_train(pl, g[0], g[1], g[2], out, stream=stream)
        tte.tt_emb_backward_sgd(pl, tok, g[0], g[1], g[2], gout, p.lr, stream=stream)
        return pl

    def timed(fn):
        for _ in range(args.warmup):
            pl = fn()
        torch.cuda.synchronize()
        assert tte.tt_emb_get_error(pl) == 0
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / args.steps

    ms_cached = timed(step_cached)
    ms_plain = timed(step_plain)
    print(json.dumps({
        "metric": f"pooled bags/s, TT-EmbeddingBag training step at batch {B} with a hot-row cache",
        "value": round(B / (ms_cached * 1e-3), 1), "unit": "bags/s", "n_gpus": 1, "higher_is_better": True,
        "dtype": "f32", "data": "synthetic (seeded Zipf/Poisson indices, Gaussian cores)",
        "config": {"workload": "skew11m-train, one step after another on one stream", "hot_rows": n_hot,
                   "lookups_served_by_cache": round(served, 4)},
        "ms_per_step_cached": round(ms_cached, 4), "ms_per_step_uncached": round(ms_plain, 4),
    }))


def kernel_source_hash() -> str:
    """sha256 prefix over every kernel source file (sorted by name)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def kernel_traffic():
    """HBM bytes per launch of each kernel from the committed counter passes,
    or {} when the kernel sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return {}
    if rec.get("source_hash") != kernel_source_hash():
        return {}
    return {k: v["fetch_bytes"] + v["write_bytes"] for k, v in rec.get("kernels", {}).items()}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; "
              "rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.forward_workload:
        forward_only(args)
        return
    if args.hot_rows > 0:
        hot_rows_step(args)
        return

    import numpy as np
    import torch

    import tensor_train_compressed_amd as tte
    import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    p = wl.make("train11m")
    t = p.tables[0]
    n1, n2, n3 = t.n
    R, D = t.rank, t.dim
    B, L = p.batch, p.L
    tabs = tte.make_tables(p.tables, p.goff)
    g = [torch.from_numpy(x).to(dev) for x in (p.g1, p.g2, p.g3)]
    dg = [torch.empty_like(x) for x in g]
    idx = torch.from_numpy(p.indices).to(dev)
    off = torch.from_numpy(p.offsets).to(dev)
    gout = torch.from_numpy(p.grad_out).to(dev)
    out = torch.empty((B, D), dtype=torch.float32, device=dev)
    # two workspaces: a batch's plan is built while the previous batch computes
    nws = tte.tt_emb_workspace_bytes(tabs, L, B, args.chunk)
    wss = [torch.empty(nws, dtype=torch.uint8, device=dev) for _ in range(2)]
    ws = wss[0]
    stream = torch.cuda.current_stream()
    pstream = torch.cuda.Stream()   # default priority, like the compute stream

    def plan():
        return tte.tt_emb_plan(tabs, idx, off, B, args.chunk, workspace=ws, stream=stream)

    def step():
        pl = plan()
        tok = tte.tt_emb_forward_train(pl, g[0], g[1], g[2], out, stream=stream)
        tte.tt_emb_backward_sgd(pl, tok, g[0], g[1], g[2], gout, p.lr, stream=stream)
        return pl

    def steps_pipelined(k):
        """k steps; the plan of step i+1 on pstream (workspace (i+1) mod 2)
        overlaps step i's forward and backward on the compute stream."""
        planned = [torch.cuda.Event(), torch.cuda.Event()]
        used = [torch.cuda.Event(), torch.cuda.Event()]
        plans = [None, None]
        pstream.wait_stream(stream)
        plans[0] = tte.tt_emb_plan(tabs, idx, off, B, args.chunk, workspace=wss[0], stream=pstream)
        planned[0].record(pstream)
        for i in range(k):
            c, n = i % 2, (i + 1) % 2
            stream.wait_event(planned[c])
            tok = tte.tt_emb_forward_train(plans[c], g[0], g[1], g[2], out, stream=stream)
            tte.tt_emb_backward_sgd(plans[c], tok, g[0], g[1], g[2], gout, p.lr, stream=stream)
            used[c].record(stream)
            if i + 1 < k:
                if i >= 1:
                    pstream.wait_event(used[n])   # workspace n: step i-1's, done
                plans[n] = tte.tt_emb_plan(tabs, idx, off, B, args.chunk, workspace=wss[n], stream=pstream)
                planned[n].record(pstream)
        return plans[(k - 1) % 2]

    pl = steps_pipelined(args.warmup)
    for _ in range(args.warmup):
        pl = step()
    torch.cuda.synchronize()
    assert tte.tt_emb_get_error(pl) == 0
    U, NC = tte.tt_emb_plan_counts(pl)

    # the timed region: exactly `steps` whole steps, synchronised on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pl = steps_pipelined(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert tte.tt_emb_get_error(pl) == 0
    ms_per_step = 1e3 * elapsed / args.steps
    bags_per_s = B * args.steps / elapsed
    # the same steps one after another on one stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pl = step()
    torch.cuda.synchronize()
    ms_per_step_serial = 1e3 * (time.perf_counter() - t0) / args.steps

    # per-call phase times: HIP events on the kernels' stream around
    # back-to-back calls (host launch gaps overlap the GPU work)
    def per_call_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = args.phase_reps
    plan_ms = per_call_ms(plan, reps)
    pl = plan()
    fwd_ms = per_call_ms(lambda: tte.tt_emb_forward(pl, g[0], g[1], g[2], out, stream=stream), reps)
    fwd_train_ms = per_call_ms(lambda: tte.tt_emb_forward_train(pl, g[0], g[1], g[2], out, stream=stream),
                               reps)
    # the backward as the step runs it: after forward_train, reusing the kept
    # P (each call consumes the kept products, so every backward follows its
    # own training forward; events bracket the backward alone)
    def bwd_after_fwd_train_ms(reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            tok = tte.tt_emb_forward_train(pl, g[0], g[1], g[2], out, stream=stream)
            e0.record(stream)
            tte.tt_emb_backward_kept(pl, tok, g[0], g[1], g[2], gout, dg[0], dg[1], dg[2], stream=stream)
            e1.record(stream)
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps

    bwd_ms = bwd_after_fwd_train_ms(reps)
    # the backward that forms P again (no kept products): the checkpoint's worth
    bwd_recompute_ms = per_call_ms(lambda: tte.tt_emb_backward(pl, g[0], g[1], g[2], gout, dg[0], dg[1], dg[2],
                                                               stream=stream), reps)
    sgd_ms = per_call_ms(lambda: tte.tt_emb_sgd(pl, g[0], g[1], g[2], dg[0], dg[1], dg[2], p.lr,
                                                stream=stream), reps)

    # the fused backward + SGD step as the timed step runs it
    def bwd_sgd_ms(reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            tok = tte.tt_emb_forward_train(pl, g[0], g[1], g[2], out, stream=stream)
            e0.record(stream)
            tte.tt_emb_backward_sgd(pl, tok, g[0], g[1], g[2], gout, p.lr, stream=stream)
            e1.record(stream)
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps

    bwd_sgd = bwd_sgd_ms(reps)
    torch.cuda.synchronize()

    # per-kernel times, measured live: the library brackets every kernel it
    # launches with HIP events on the stream it launches it on
    # (tt_emb_set_timing); one instrumented pass of `reps` whole steps and
    # `reps` plain forward calls on the same inputs, after the timed region
    def kernel_avgs(records, calls):
        agg = {}
        for k, ms in records:
            agg.setdefault(k, []).append(ms)
        return {k: {"us": 1e3 * sum(v) / len(v), "per_call": len(v) / calls} for k, v in agg.items()}

    tte.tt_emb_set_timing(None, True)
    recs = []
    for _ in range(reps):
        recs += tte.tt_emb_kernel_times(step(), stream)
    tte.tt_emb_set_timing(None, False)
    step_kernels = kernel_avgs(recs, reps)
    pl = plan()
    tte.tt_emb_set_timing(pl, True)
    for _ in range(reps):
        tte.tt_emb_forward(pl, g[0], g[1], g[2], out, stream=stream)
    fwd_kernels = kernel_avgs(tte.tt_emb_kernel_times(pl, stream), reps)
    tte.tt_emb_set_timing(pl, False)

    # executed work (distinct rows of a group are contracted once)
    key_i3, row_n = np.unique(p.indices, return_counts=True)   # one table: a distinct index is a row run
    U_row = int(key_i3.size)
    U_one = int((row_n == 1).sum())         # runs of one lookup: no S row (their grad row serves)
    pre = U * 2 * n1 * n2 * R * R            # prefix products, per call
    suf = U_row * 2 * n1 * n2 * n3 * R       # one suffix-sized product per distinct row
    core_elems = p.g1.size + p.g2.size + p.g3.size
    # kernel -> (fp32 FLOP, fp64 FLOP, algorithmic HBM bytes) per launch; the
    # bytes count each datum once (a gathered row that many lookups share is
    # read from HBM once at best; its other reads hit L2 or the Infinity
    # Cache), and `gathered` below gives the per-lookup row reads
    work = {
        "k_fwd_batch": (pre + suf, 0, 0), "k_fwd_batch_keep": (pre + suf, 0, 0),
        # stage rows of the distinct rows, run ids, offsets in; pooled rows out
        "k_pool": (L * D, 0, 4 * U_row * D + 4 * L + 8 * (B + 1) + 4 * B * D),
        # grad rows, sorted bags / run ids / keys in; S rows of the runs of
        # more than one lookup out
        "k_bwd_sum": (0, L * D, 4 * B * D + 12 * L + 4 * (U_row - U_one) * D),
        "k_bwd_runs_c3": (suf, suf, 0),
        # dG3 (c3 row sums), dG1 and dG2 in one launch
        "k_bwd_dg123": (0, 2 * pre + U_row * R * n3, 0),
        "k_sgd": (2 * core_elems, 0, 12 * core_elems),
    }
    PEAK_FP64_TFLOPS = 78.6
    gathered = {"k_pool": 4 * L * D, "k_bwd_sum": 4 * L * D}

    def kernel_roofline(name, rec):
        f32, f64, by = work.get(name, (0, 0, 0))
        sec = rec["us"] * 1e-6
        out_ = {"kernel": name, "us": round(rec["us"], 2), "launches_per_call": rec["per_call"]}
        tb = traffic_of(name)
        if tb is not None:
            # measured HBM bytes (counters) over the event-timed launch
            out_["traffic"] = tb
            out_["hbm_frac_measured"] = round(tb / sec / 1e9 / PEAK_HBM_GBS, 4)
        if f32 or f64:
            out_["fp32_tflops"] = round(f32 / sec / 1e12, 2)
            out_["fp64_tflops"] = round(f64 / sec / 1e12, 2)
            out_["frac"] = round(f32 / sec / 1e12 / PEAK_FP32_TFLOPS + f64 / sec / 1e12 / PEAK_FP64_TFLOPS, 4)
            out_["bound"] = "mfma"
        if by and not (f32 > 1e9 or f64 > 1e9):
            out_["bound"] = "hbm"
            out_["gbs"] = round(by / sec / 1e9, 1)
            out_["frac"] = round(by / sec / 1e9 / PEAK_HBM_GBS, 4)
        if name in gathered:
            # one D-row read per lookup, most from L2 / the Infinity Cache
            out_["gathered_row_gbs"] = round(gathered[name] / sec / 1e9, 1)
        return out_

    kb = fwd_kernels["k_fwd_batch"]["us"] * 1e-6
    kpool = fwd_kernels["k_pool"]["us"] * 1e-6
    achieved_tflops = (pre + suf) / kb / 1e12
    fwd_flop = pre + suf + L * D
    fwd_flop_per_lookup = pre + L * (2 * n1 * n2 * n3 * R + D)
    core_bytes = 4 * core_elems
    fwd_bytes = 8 * L + 8 * (B + 1) + core_bytes + 4 * B * D
    traffic_by_kernel = kernel_traffic()

    def traffic_of(name):
        """Counter bytes of the kernel a timing record names (the training
        forward's batch kernel is the KEEP instantiation)."""
        for k, v in traffic_by_kernel.items():
            base = k.split("<")[0]
            if name == "k_fwd_batch_keep":
                if base == "k_fwd_batch" and k.rstrip(">").endswith("true"):
                    return v
            elif name == "k_fwd_batch":
                if base == "k_fwd_batch" and k.rstrip(">").endswith("false"):
                    return v
            elif base == name:
                return v
        return None

    traffic = traffic_of("k_fwd_batch")
    step_rows = sorted((kernel_roofline(k, v) for k, v in step_kernels.items()),
                       key=lambda r: -r["us"] * r["launches_per_call"])
    step_kernel_ms = sum(r["us"] * r["launches_per_call"] for r in step_rows) * 1e-3
    f32_step = sum(work.get(k, (0, 0, 0))[0] * v["per_call"] for k, v in step_kernels.items())
    f64_step = sum(work.get(k, (0, 0, 0))[1] * v["per_call"] for k, v in step_kernels.items())

    if args.calibrate_copy:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter values
        # scale the counters of the forward kernels to bytes
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if args.cpu_bags > 0:
        cpu = cpu_baseline(p, args.cpu_bags, args.chunk)

    rec = {
        "metric": "pooled bags/s, TT-EmbeddingBag plan+forward+backward+SGD step at batch 32768",
        "value": round(bags_per_s, 1),
        "unit": "bags/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_serial": round(ms_per_step_serial, 4),
        "schedule": "next batch's plan on a second stream (two workspaces), overlapping this batch's "
                    "forward and backward; forward after the previous step's SGD",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Zipf/Poisson indices, Gaussian cores)",
        "config": {"workload": "skew11m-train: 11M rows 200x220x250, dim 128=4x8x4, rank 32, "
                               "B=32768 Poisson(20) clip[1,100], Zipf(1.1) unpermuted, "
                               "plan+fwd+bwd+SGD lr 0.01",
                   "global_batch": B, "lookups": L, "prefix_groups": U, "distinct_rows": U_row,
                   "chunks": NC, "chunk": args.chunk},
        "phases_ms_per_call": {"plan": round(plan_ms, 4), "forward": round(fwd_ms, 4),
                               "forward_train": round(fwd_train_ms, 4),
                               "backward_after_forward_train": round(bwd_ms, 4),
                               "backward_forming_p_again": round(bwd_recompute_ms, 4),
                               "sgd": round(sgd_ms, 4),
                               "backward_sgd_after_forward_train": round(bwd_sgd, 4)},
        "forward_bags_per_s": round(B / (fwd_ms * 1e-3), 1),
        "plan_forward_bags_per_s": round(B / ((plan_ms + fwd_ms) * 1e-3), 1),
        "forward_rows_per_s": round(L / (fwd_ms * 1e-3), 1),
        "workspace_bytes": int(ws.numel()),
        "workspaces": len(wss),
        "roofline": {"kernel": "k_fwd_batch (the forward's dominant kernel: prefix and suffix products)",
                     "bound": "mfma", "achieved": round(achieved_tflops, 3),
                     "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / PEAK_FP32_TFLOPS, 4),
                     "traffic": traffic,
                     "avg_launch_us": round(kb * 1e6, 2),
                     "flop_per_launch": int(pre + suf),
                     "flop_per_launch_if_every_lookup_contracted": int(pre + L * 2 * n1 * n2 * n3 * R)},
        "roofline_forward_call": {"kernels": "k_fwd_batch + k_pool", "us": round((kb + kpool) * 1e6, 2),
                                  "flop": int(fwd_flop), "flop_if_every_lookup_contracted": int(fwd_flop_per_lookup),
                                  "achieved": round(fwd_flop / (kb + kpool) / 1e12, 3), "unit": "TFLOP/s",
                                  "frac": round(fwd_flop / (kb + kpool) / 1e12 / PEAK_FP32_TFLOPS, 4),
                                  "algorithmic_bytes": int(fwd_bytes),
                                  "hbm_frac_algorithmic": round(fwd_bytes / (kb + kpool) / 1e9 / PEAK_HBM_GBS, 4)},
        "roofline_step": {"kernel_ms_per_step": round(step_kernel_ms, 4),
                          "fp32_flop": int(f32_step), "fp64_flop": int(f64_step),
                          "fp32_frac": round(f32_step / (step_kernel_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4),
                          "fp64_frac": round(f64_step / (step_kernel_ms * 1e-3) / 1e12 / PEAK_FP64_TFLOPS, 4),
                          "kernels": step_rows},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(p, nbags: int, chunk: int):
    """The CPU oracle (plan, forward, backward, SGD) on the first `nbags` bags
    of the same batch; bags/s over that sample."""
    import oracle
    import workloads as wl

    nb = min(nbags, p.batch)
    Ls = int(p.offsets[nb])
    sub = wl.Problem(p.name, p.tables, nb, p.g1.copy(), p.g2.copy(), p.g3.copy(), p.goff,
                     p.indices[:Ls], p.offsets[:nb + 1].copy(), p.grad_out[:nb], p.lr)
    t0 = time.perf_counter()
    oracle.plan_problem(sub, chunk)
    oracle.forward_problem(sub)
    d = oracle.backward_problem(sub)
    for c, x in zip((sub.g1, sub.g2, sub.g3), d):
        oracle.sgd(c, x, sub.lr)
    el = time.perf_counter() - t0
    return {"value": round(nb / el, 3), "unit": "bags/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(el, 3),
            "sample": f"first {nb} bags ({Ls} lookups) of the same batch: numpy plan, "
                      f"fp64 C forward + backward (OpenMP), SGD"}


if __name__ == "__main__":
    main()
