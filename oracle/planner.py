"""Planner oracle: the canonical integer tables of prefix grouping, in NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages describe the task-formation step only in words: lookups that share
high-order TT core indices are grouped so that the shared part of the chain is
done once ("FlowTT: Exploiting Computation Flow Reuse in Irregular
Tensor-Train Embedding", summary card, key innovations: prefix-based index
grouping; abstract: flow-aligned prefix-based index grouping), and skewed
groups are cut into chunks that persistent threads steal (same passages:
dynamic load balancing, chunk-based work stealing). Which lookups form a group
is fixed by that description; the order of groups, the order inside a group
and the chunk size are not. The readings taken here, which make every table
unique:

  split    i3 = idx mod m3, i2 = (idx div m3) mod m2, i1 = idx div (m2*m3)
           (i1 most significant, so (i1, i2) are the high-order digits)
  key      base_t + i2*m1 + i1, base_t = sum over earlier tables of m1*m2:
           one key per (table, i1, i2) prefix; groups sharing a G2 slice
           (same table and i2) get adjacent keys
  order    lookups sorted by (key, i3), ties kept in increasing lookup id:
           inside a group, lookups of the same table row are adjacent, so a
           row that occurs several times is contracted once (the pages' point
           that prefix grouping removes redundant core operations extends to
           the last core when whole rows repeat)
  groups   maximal runs of equal key in sorted order
  chunks   each group, in order, cut into consecutive pieces of exactly C
           lookups; only a group's last piece may be shorter; no piece spans
           two groups

Every table is int32, as on the GPU.
"""
from __future__ import annotations

from typing import Dict, Sequence, Tuple

import numpy as np


class PlanError(ValueError):
    pass


def bag_of_lookups(offsets: np.ndarray, L: int) -> np.ndarray:
    """bag_of[l] = the q with offsets[q] <= l < offsets[q+1]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    if offsets.size < 1 or offsets[0] != 0 or offsets[-1] != L or np.any(np.diff(offsets) < 0):
        raise PlanError("offsets must start at 0, end at L and be non-decreasing")
    lens = np.diff(offsets)
    return np.repeat(np.arange(lens.size, dtype=np.int64), lens)


def plan(radices: Sequence[Tuple[int, int, int]], num_rows: Sequence[int], B: int,
         indices: np.ndarray, offsets: np.ndarray, chunk: int) -> Dict[str, np.ndarray]:
    """Return the planner's tables for T = len(radices) tables of B bags each."""
    if chunk < 1:
        raise PlanError("chunk must be >= 1")
    T = len(radices)
    idx = np.asarray(indices, dtype=np.int64)
    L = idx.size
    if np.asarray(offsets).size != T * B + 1:
        raise PlanError("offsets must have T*B+1 entries")
    bag = bag_of_lookups(offsets, L)
    t = bag // B if B > 0 else np.zeros(0, np.int64)

    m = np.asarray(radices, dtype=np.int64).reshape(T, 3)
    N = np.asarray(num_rows, dtype=np.int64)
    if np.any(idx < 0) or np.any(idx >= N[t]):
        raise PlanError("index out of range")
    m1, m2, m3 = m[t, 0], m[t, 1], m[t, 2]
    i3 = idx % m3
    i2 = (idx // m3) % m2
    i1 = idx // (m2 * m3)
    base = np.concatenate([[0], np.cumsum(m[:, 0] * m[:, 1])])
    key = base[t] + i2 * m1 + i1

    M3 = int(m[:, 2].max())
    perm = np.argsort(key * M3 + i3, kind="stable")
    skey = key[perm]
    if L:
        first = np.concatenate([[True], skey[1:] != skey[:-1]])
        gstart = np.flatnonzero(first)
    else:
        gstart = np.zeros(0, np.int64)
    group_key = skey[gstart]
    group_start = np.concatenate([gstart, [L]])

    cg, cb, ce = [], [], []
    for g in range(group_key.size):
        s, e = int(group_start[g]), int(group_start[g + 1])
        for b in range(s, e, chunk):
            cg.append(g); cb.append(b); ce.append(min(b + chunk, e))

    i32 = lambda a: np.asarray(a, dtype=np.int64).astype(np.int32)
    return {
        "bag_of": i32(bag), "i1": i32(i1), "i2": i32(i2), "i3": i32(i3), "key": i32(key),
        "perm": i32(perm), "sorted_i3": i32(i3[perm]), "sorted_bag": i32(bag[perm]),
        "group_key": i32(group_key), "group_start": i32(group_start),
        "chunk_group": i32(cg), "chunk_begin": i32(cb), "chunk_end": i32(ce),
        "key_space": np.int64(base[-1]),
    }


def plan_problem(p, chunk: int) -> Dict[str, np.ndarray]:
    """plan() on a workloads.Problem."""
    return plan([t.m for t in p.tables], [t.num_rows for t in p.tables], p.batch,
                p.indices, p.offsets, chunk)
