#!/usr/bin/env python3
"""Benchmark of the TT-EmbeddingBag hot path on one MI355X.

Workload: one 11,000,000-row table (radices 200x220x250), dim 128 (4x8x4),
TT rank 32, fp32 cores; a batch of 32,768 bags with Poisson(20) lengths
clipped to [1,100] and unpermuted Zipf(1.1) indices; grad_out ~ N(0,1) and an
SGD step with lr 0.01. One step is the whole path on one batch: plan (split,
prefix grouping, chunking), forward, backward, SGD, with every input already
resident in HBM.

Prints one JSON line: whole-step pooled bags/s as `value`, plus per-phase
times from HIP events, the forward kernel's roofline figures, and the CPU
oracle timed on a bounded sample of the same batch as `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3      # MI355X published dense FP32 (vector and matrix)
PEAK_HBM_GBS = 8000.0         # MI355X published HBM3E bandwidth


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--chunk", type=int, default=256)
    ap.add_argument("--cpu-bags", type=int, default=256,
                    help="bags of the batch the CPU oracle baseline runs on (0: skip)")
    ap.add_argument("--phase-reps", type=int, default=20)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(see the sharding notes in DESIGN.md); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

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
    g_init = [torch.from_numpy(x).to(dev) for x in (p.g1, p.g2, p.g3)]
    g = [x.clone() for x in g_init]
    dg = [torch.empty_like(x) for x in g]
    idx = torch.from_numpy(p.indices).to(dev)
    off = torch.from_numpy(p.offsets).to(dev)
    gout = torch.from_numpy(p.grad_out).to(dev)
    out = torch.empty((B, D), dtype=torch.float32, device=dev)
    ws = torch.empty(tte.tt_emb_workspace_bytes(tabs, L, B, args.chunk), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def step():
        pl = tte.tt_emb_plan(tabs, idx, off, B, args.chunk, workspace=ws, stream=stream)
        tte.tt_emb_forward(pl, g[0], g[1], g[2], out, stream=stream)
        tte.tt_emb_backward(pl, g[0], g[1], g[2], gout, dg[0], dg[1], dg[2], stream=stream)
        tte.tt_emb_sgd(pl, g[0], g[1], g[2], dg[0], dg[1], dg[2], p.lr, stream=stream)
        return pl

    for _ in range(args.warmup):
        pl = step()
    torch.cuda.synchronize()
    assert tte.tt_emb_get_error(pl) == 0
    U, NC = tte.tt_emb_plan_counts(pl)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pl = step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    bags_per_s = B * args.steps / elapsed

    # per-phase HIP events on the stream the kernels run on
    reps = args.phase_reps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(reps)]
    for r in range(reps):
        e = ev[r]
        e[0].record(stream)
        pl = tte.tt_emb_plan(tabs, idx, off, B, args.chunk, workspace=ws, stream=stream)
        e[1].record(stream)
        tte.tt_emb_forward(pl, g[0], g[1], g[2], out, stream=stream)
        e[2].record(stream)
        tte.tt_emb_backward(pl, g[0], g[1], g[2], gout, dg[0], dg[1], dg[2], stream=stream)
        e[3].record(stream)
        tte.tt_emb_sgd(pl, g[0], g[1], g[2], dg[0], dg[1], dg[2], p.lr, stream=stream)
        e[4].record(stream)
    torch.cuda.synchronize()
    ph = np.array([[ev[r][k].elapsed_time(ev[r][k + 1]) for k in range(4)] for r in range(reps)])
    plan_ms, fwd_ms, bwd_ms, sgd_ms = (float(np.median(ph[:, k])) for k in range(4))

    # algorithmic work of one forward launch (prefix per group, suffix + pool per lookup)
    fwd_flop = U * 2 * n1 * n2 * R * R + L * (2 * n1 * n2 * n3 * R + D)
    touched = len(np.unique(p.indices // t.m[2]))  # not used for flops; cores are tiny
    core_bytes = 4 * (p.g1.size + p.g2.size + p.g3.size)
    fwd_bytes = 8 * L + 8 * (B + 1) + core_bytes + 4 * B * D
    achieved_tflops = fwd_flop / (fwd_ms * 1e-3) / 1e12
    del touched

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
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Zipf/Poisson indices, Gaussian cores)",
        "config": {"workload": "skew11m-train: 11M rows 200x220x250, dim 128=4x8x4, rank 32, "
                               "B=32768 Poisson(20) clip[1,100], Zipf(1.1) unpermuted, "
                               "fwd+bwd+SGD lr 0.01",
                   "global_batch": B, "lookups": L, "prefix_groups": U, "chunks": NC,
                   "chunk": args.chunk},
        "phases_ms": {"plan": round(plan_ms, 4), "forward": round(fwd_ms, 4),
                      "backward": round(bwd_ms, 4), "sgd": round(sgd_ms, 4)},
        "forward_bags_per_s": round(B / (fwd_ms * 1e-3), 1),
        "plan_forward_bags_per_s": round(B / ((plan_ms + fwd_ms) * 1e-3), 1),
        "forward_rows_per_s": round(L / (fwd_ms * 1e-3), 1),
        "roofline": {"kernel": "tt_emb_forward (output zero-fill + k_fwd)",
                     "bound": "alu", "achieved": round(achieved_tflops, 3),
                     "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / PEAK_FP32_TFLOPS, 4),
                     "algorithmic_flop": int(fwd_flop), "algorithmic_bytes": int(fwd_bytes),
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(p, nbags: int, chunk: int):
    """The CPU oracle (plan, forward, backward, SGD) on the first `nbags` bags
    of the same batch; bags/s over that sample."""
    import numpy as np

    import oracle
    import workloads as wl

    nb = min(nbags, p.batch)
    Ls = int(p.offsets[nb])
    sub = wl.Problem(p.name, p.tables, nb, p.g1, p.g2, p.g3, p.goff, p.indices[:Ls],
                     p.offsets[:nb + 1].copy(), p.grad_out[:nb], p.lr)
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
