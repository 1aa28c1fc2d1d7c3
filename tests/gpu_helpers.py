"""Helpers for the GPU tests: move a workloads.Problem to the device and run
the library through its Python binding (which calls the C ABI)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import tensor_train_compressed_amd as tte

DEV = "cuda:0"


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


class DevProblem:
    def __init__(self, p, chunk=256):
        self.p = p
        self.chunk = chunk
        self.tables_c = tte.make_tables(p.tables, p.goff)
        self.g1 = torch.from_numpy(p.g1).to(DEV)
        self.g2 = torch.from_numpy(p.g2).to(DEV)
        self.g3 = torch.from_numpy(p.g3).to(DEV)
        self.idx = torch.from_numpy(np.ascontiguousarray(p.indices)).to(DEV)
        self.off = torch.from_numpy(np.ascontiguousarray(p.offsets)).to(DEV)
        self.TB = p.T * p.batch
        self.D = p.dim
        self.gout = None if p.grad_out is None else torch.from_numpy(p.grad_out).to(DEV)
        self.plan = None

    def make_plan(self):
        self.plan = tte.tt_emb_plan(self.tables_c, self.idx, self.off, self.p.batch, self.chunk)
        return self.plan

    def forward(self):
        if self.plan is None:
            self.make_plan()
        out = torch.empty((self.TB, self.D), dtype=torch.float32, device=DEV)
        tte.tt_emb_forward(self.plan, self.g1, self.g2, self.g3, out)
        return out

    def backward(self):
        if self.plan is None:
            self.make_plan()
        d1 = torch.empty_like(self.g1)
        d2 = torch.empty_like(self.g2)
        d3 = torch.empty_like(self.g3)
        tte.tt_emb_backward(self.plan, self.g1, self.g2, self.g3, self.gout, d1, d2, d3)
        return d1, d2, d3

    def plan_tables(self):
        """Planner tables copied to host numpy (synchronises)."""
        pl = self.plan
        L = self.p.L
        U, NC = tte.tt_emb_plan_counts(pl)
        get = lambda name, n: tte.plan_table(pl, name, n).cpu().numpy().copy()
        return {
            "key": get("key", L), "i3": get("i3", L), "bag_of": get("bag_of", L),
            "perm": get("perm", L), "sorted_i3": get("sorted_i3", L),
            "sorted_bag": get("sorted_bag", L), "group_key": get("group_key", U),
            "group_start": get("group_start", U + 1), "chunk_group": get("chunk_group", NC),
            "chunk_begin": get("chunk_begin", NC), "chunk_end": get("chunk_end", NC),
        }


def assert_close(got, ref, what, tol=1e-4):
    """|got - ref| <= tol * (1 + |ref|) elementwise (ref in float64)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = tol * (1.0 + np.abs(ref))
    bad = err > bound
    if np.any(bad):
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} err {err[i]:.3e} bound {bound[i]:.3e}")
    return float(np.max(err / (1.0 + np.abs(ref)))) if err.size else 0.0
