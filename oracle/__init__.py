"""CPU oracle for the sum-pooled Tensor-Train embedding gather.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product (the HIP library and its
Python binding) never imports, links or calls anything here, and nothing here
imports the product: the two share no code. Both sides only share the seeded
input generators in `workloads`, which hold none of the method's arithmetic.

Contents:
  tt_oracle.c  plain C, fp64: per-lookup TT chain, sum pooling, core gradients
  planner.py   NumPy: index split, stable prefix-key sort, groups, chunks
  this file    ctypes loader and NumPy-facing wrappers; SGD by its definition

Parity status of each function (pins live in tests/, marked "not gpu"):
  forward      pinned: brute-force table materialisation in another
               contraction order, rank-1 Kronecker closed form, gauge
               invariance, multilinearity and pooling additivity
  backward     pinned: exact adjoint identity against the forward oracle,
               brute-force chain rule on tiny shapes, rank-1 closed form
  sgd          pinned by its arithmetic definition on hand-made values
  cache        (hot-row cache) pinned: an empty hot set changes nothing; a hot
               set holding the rows' own TT values reproduces the plain
               forward; the adjoint identity for dW against the forward; the
               cores' gradients add up with those of the hot lookups alone to
               the plain backward
  planner      pinned: exact digit identity over every row of a table,
               pure-Python brute-force stable sort on small inputs, and the
               partition invariants of groups and chunks
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence, Tuple

import numpy as np

from . import planner  # noqa: F401  (re-exported)
from .planner import PlanError, plan, plan_problem  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tt_oracle.c")
_LIB = os.environ.get("TT_ORACLE_LIB") or os.path.join(_HERE, "libtt_oracle.so")
_lock = threading.Lock()
_lib = None

OK, BAD_ARG, BAD_INDEX, BAD_OFFSETS, NO_MEMORY = 0, -1, -2, -3, -4

# AddressSanitizer + UndefinedBehaviorSanitizer build (gcc); the process that
# loads it must preload gcc's libasan (LD_PRELOAD) and set TT_ORACLE_LIB.
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


class OracleError(RuntimeError):
    pass


def build(force: bool = True, sanitize: bool = False, out: Optional[str] = None) -> str:
    """Compile tt_oracle.c with gcc (OpenMP) into oracle/libtt_oracle.so (-O2),
    or, with sanitize=True, an ASan/UBSan build into `out`."""
    lib = out or _LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + f".tmp{os.getpid()}"
        opt = SANITIZE_FLAGS if sanitize else ["-O2"]
        subprocess.run(["gcc", *opt, "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-o", tmp, _SRC], check=True)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.environ.get("TT_ORACLE_LIB"):
                build(force=False)
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i32, i64 = ctypes.c_int32, ctypes.c_int64
            lib.tto_forward.argtypes = [i32, P, P, P, P, P, P, P, P, P, P, i64, i64, P, i64, P]
            lib.tto_forward.restype = ctypes.c_int
            lib.tto_backward.argtypes = [i32, P, P, P, P, P, P, P, P, P, P, i64, i64, P, P,
                                         P, i64, P, i64, P, i64]
            lib.tto_backward.restype = ctypes.c_int
            lib.tto_num_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS or all cores)."""
    return int(_load().tto_num_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _tables(tables) -> Tuple[np.ndarray, ...]:
    N = np.ascontiguousarray([t.num_rows for t in tables], dtype=np.int64)
    m = np.ascontiguousarray([t.m for t in tables], dtype=np.int64).reshape(-1)
    n = np.ascontiguousarray([t.n for t in tables], dtype=np.int64).reshape(-1)
    R = np.ascontiguousarray([t.rank for t in tables], dtype=np.int64)
    return N, m, n, R


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(f"{what}: oracle returned {rc}")


def forward(tables: Sequence, g1, g2, g3, goff, indices, offsets, B: int,
            bags: Optional[np.ndarray] = None) -> np.ndarray:
    """Pooled outputs (float64) of the listed bags (all bags if None)."""
    lib = _load()
    N, m, n, R = _tables(tables)
    goff = np.ascontiguousarray(goff, dtype=np.int64).reshape(-1)
    g1, g2, g3 = (np.ascontiguousarray(x, dtype=np.float32) for x in (g1, g2, g3))
    idx = np.ascontiguousarray(indices, dtype=np.int64)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    D = tables[0].n[0] * tables[0].n[1] * tables[0].n[2]
    if bags is not None:
        bags = np.ascontiguousarray(bags, dtype=np.int64)
        nb = bags.size
    else:
        nb = len(tables) * B
    out = np.empty((nb, D), dtype=np.float64)
    rc = lib.tto_forward(len(tables), _ptr(N), _ptr(m), _ptr(n), _ptr(R), _ptr(goff),
                         _ptr(g1), _ptr(g2), _ptr(g3), _ptr(idx), _ptr(off), idx.size, B,
                         _ptr(bags), nb, _ptr(out))
    _check(rc, "forward")
    return out


def backward(tables: Sequence, g1, g2, g3, goff, indices, offsets, B: int, grad_out,
             mask: Optional[np.ndarray] = None):
    """(dG1, dG2, dG3) in float64, same packing as the cores; only lookups
    with mask[l] != 0 contribute (all if mask is None)."""
    lib = _load()
    N, m, n, R = _tables(tables)
    goff = np.ascontiguousarray(goff, dtype=np.int64).reshape(-1)
    g1, g2, g3 = (np.ascontiguousarray(x, dtype=np.float32) for x in (g1, g2, g3))
    idx = np.ascontiguousarray(indices, dtype=np.int64)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    go = np.ascontiguousarray(grad_out, dtype=np.float32)
    mk = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    d1 = np.empty(g1.size, np.float64)
    d2 = np.empty(g2.size, np.float64)
    d3 = np.empty(g3.size, np.float64)
    rc = lib.tto_backward(len(tables), _ptr(N), _ptr(m), _ptr(n), _ptr(R), _ptr(goff),
                          _ptr(g1), _ptr(g2), _ptr(g3), _ptr(idx), _ptr(off), idx.size, B,
                          _ptr(go), _ptr(mk), _ptr(d1), d1.size, _ptr(d2), d2.size,
                          _ptr(d3), d3.size)
    _check(rc, "backward")
    return d1, d2, d3


def sgd(g: np.ndarray, dg: np.ndarray, lr: float) -> np.ndarray:
    """Plain SGD step G <- G - lr * dG, in float64."""
    return np.asarray(g, dtype=np.float64) - float(lr) * np.asarray(dg, dtype=np.float64)


def forward_problem(p, bags=None) -> np.ndarray:
    return forward(p.tables, p.g1, p.g2, p.g3, p.goff, p.indices, p.offsets, p.batch, bags)


def backward_problem(p, mask=None):
    return backward(p.tables, p.g1, p.g2, p.g3, p.goff, p.indices, p.offsets, p.batch,
                    p.grad_out, mask)


# ---------------------------------------------------------------------------
# Hot-row cache (TT-Rec abstract: caching strategies for the embedding
# lookups; TT-Rec news article, method paragraph: a cache structure that uses
# the skewed, sparse feature distribution and changes accuracy). Reading: a
# set of hot rows per table is kept uncompressed, as trainable vectors W[s];
# a lookup of a hot row takes W[s] in place of the TT contraction, its grad
# row goes to dW[s], and the TT cores get gradients from the other lookups
# only. Hot entry s is the pair (hot_table[s], hot_row[s]); when a pair is
# listed twice its first slot serves it (the later slot gets no lookups).

def _bag_of(offsets: np.ndarray, L: int) -> np.ndarray:
    off = np.asarray(offsets, dtype=np.int64)
    return np.repeat(np.arange(off.size - 1, dtype=np.int64), np.diff(off))[:L]


def cache_slots(p, hot_table, hot_row) -> np.ndarray:
    """Slot of every lookup's row in the hot set (int64 [L]; -1: not hot)."""
    bag = _bag_of(p.offsets, p.L)
    t = bag // p.batch
    key = t * (np.int64(1) << 40) + np.asarray(p.indices, dtype=np.int64)
    hk = np.asarray(hot_table, dtype=np.int64) * (np.int64(1) << 40) + np.asarray(hot_row, dtype=np.int64)
    if hk.size == 0:
        return np.full(p.L, -1, np.int64)
    uk, first = np.unique(hk, return_index=True)   # first slot of each distinct pair
    pos = np.searchsorted(uk, key)
    pos_c = np.minimum(pos, uk.size - 1)
    hit = uk[pos_c] == key
    return np.where(hit, first[pos_c], -1).astype(np.int64)


def forward_cached(p, hot_table, hot_row, W) -> np.ndarray:
    """Pooled outputs (float64) with the hot rows taken from W [n_hot][D]."""
    slot = cache_slots(p, hot_table, hot_row)
    bag = _bag_of(p.offsets, p.L)
    cold = slot < 0
    TB = p.T * p.batch
    counts = np.bincount(bag[cold], minlength=TB)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    out = forward(p.tables, p.g1, p.g2, p.g3, p.goff, np.asarray(p.indices)[cold], off, p.batch)
    np.add.at(out, bag[~cold], np.asarray(W, dtype=np.float64)[slot[~cold]])
    return out


def backward_cached(p, hot_table, hot_row, n_hot: int):
    """(dG1, dG2, dG3, dW) in float64: the cores' gradients from the lookups
    of rows outside the hot set, and dW [n_hot][D] from the hot ones."""
    slot = cache_slots(p, hot_table, hot_row)
    bag = _bag_of(p.offsets, p.L)
    cold = slot < 0
    d1, d2, d3 = backward_problem(p, mask=cold.astype(np.uint8))
    dW = np.zeros((n_hot, p.dim), np.float64)
    np.add.at(dW, slot[~cold], np.asarray(p.grad_out, dtype=np.float64)[bag[~cold]])
    return d1, d2, d3, dW


def materialise_rows(p, hot_table, hot_row) -> np.ndarray:
    """TT rows of the listed (table, row) pairs (float64 [n][D]): the forward
    of one-lookup bags."""
    ht = np.asarray(hot_table, dtype=np.int64)
    hr = np.asarray(hot_row, dtype=np.int64)
    out = np.empty((ht.size, p.dim), np.float64)
    for t in np.unique(ht):
        sel = np.nonzero(ht == t)[0]
        tab = [p.tables[t]]
        goff = np.asarray(p.goff).reshape(-1, 3)[t:t + 1]
        o = forward(tab, p.g1, p.g2, p.g3, goff, hr[sel], np.arange(sel.size + 1, dtype=np.int64),
                    sel.size)
        out[sel] = o
    return out
