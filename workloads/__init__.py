"""Seeded synthetic inputs for the sum-pooled Tensor-Train embedding gather.

This module only draws random numbers and lays them out in the shared input
format. It holds none of the method's arithmetic (no index split, no
contraction, no grouping) and is the one piece of code that both the CPU
oracle's tests and the GPU path's tests/benchmark use.

The pages (FlowTT summary card and abstract; TT-Rec abstract) measure on
Meta's synthetic recommendation benchmarks and on Criteo via MLPerf-DLRM,
none of which are available here and whose shapes the pages do not give.
The generators below stand in for them with the shapes, value distributions
and skew of five synthetic workloads:

  tiny        1,000 rows = 10x10x10, dim 16 = 2x2x4, rank 4, cores N(0, 0.1^2),
              256 bags of one lookup, uniform indices
  table1m     1,000,000 rows = 100^3, dim 64 = 4x4x4, rank 16, 4,096 bags of
              one lookup, Zipf(1.05) ranks through a random row permutation
  skew11m     11,000,000 rows = 200x220x250, dim 128 = 4x8x4, rank 32,
              32,768 bags with Poisson(20) lengths clipped to [1,100],
              unpermuted Zipf(1.1) indices
  multi26     26 tables, rows log-uniform in [1e3, 4e7] split into three
              near-equal radices, dim 64 = 4x4x4, rank 32, 32,768 bags per
              table with unclipped Poisson(10) lengths, Zipf(alpha_t),
              alpha_t ~ U(0.8, 1.2)
  train11m    skew11m's inputs plus grad_out ~ N(0,1) and learning rate 0.01

Core init: the TT-Rec abstract recommends a "sampled Gaussian" init without
a constant; we read the "N(0, 1/sqrt(R*n))" notation as a variance, i.e.
std = (R*n_k)^(-1/4) with n_k the core's own dim factor.

Zipf is the bounded form P(k) ~ k^-alpha over k = 1..N, drawn by inverse CDF
(searchsorted on a float64 cumulative sum); the row is k-1, permuted only
where stated (table1m).

Layout shared with both sides (all numpy, host memory):
  cores  g1: float32 flat, per table [m1][n1][R]      (slice G1[i1] is n1 x R)
         g2: float32 flat, per table [m2][R][n2][R]   (slice G2[i2] is R x n2 x R)
         g3: float32 flat, per table [m3][R][n3]      (slice G3[i3] is R x n3)
  goff   int64 [T][3] element offset of each table's cores in g1/g2/g3
  indices int64 [L], offsets int64 [T*B+1] (CSR bags; bag q = t*B + b)
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Table", "Problem", "make", "make_custom", "near_equal_radices",
    "bounded_zipf", "CONFIGS",
]


@dataclasses.dataclass(frozen=True)
class Table:
    num_rows: int                 # N: valid indices are [0, N)
    m: Tuple[int, int, int]       # row radices, m1*m2*m3 >= N
    n: Tuple[int, int, int]       # dim factors, D = n1*n2*n3
    rank: int                     # R (internal ranks; boundary ranks are 1)

    @property
    def dim(self) -> int:
        return self.n[0] * self.n[1] * self.n[2]

    def core_sizes(self) -> Tuple[int, int, int]:
        m1, m2, m3 = self.m
        n1, n2, n3 = self.n
        R = self.rank
        return (m1 * n1 * R, m2 * R * n2 * R, m3 * R * n3)


@dataclasses.dataclass
class Problem:
    name: str
    tables: List[Table]
    batch: int                    # B bags per table
    g1: np.ndarray                # float32
    g2: np.ndarray
    g3: np.ndarray
    goff: np.ndarray              # int64 [T][3]
    indices: np.ndarray           # int64 [L]
    offsets: np.ndarray           # int64 [T*B+1]
    grad_out: Optional[np.ndarray] = None   # float32 [T*B][D]
    lr: Optional[float] = None

    @property
    def T(self) -> int:
        return len(self.tables)

    @property
    def L(self) -> int:
        return int(self.indices.shape[0])

    @property
    def dim(self) -> int:
        return self.tables[0].dim

    def table_arrays(self):
        """Per-table descriptor columns as int64 arrays (N, m[3], n[3], R, goff[3])."""
        N = np.array([t.num_rows for t in self.tables], dtype=np.int64)
        m = np.array([t.m for t in self.tables], dtype=np.int64).reshape(-1, 3)
        n = np.array([t.n for t in self.tables], dtype=np.int64).reshape(-1, 3)
        R = np.array([t.rank for t in self.tables], dtype=np.int64)
        return N, m, n, R, self.goff.reshape(-1, 3).astype(np.int64)


def near_equal_radices(N: int) -> Tuple[int, int, int]:
    """Three near-equal radices with m1*m2*m3 >= N, computed in exact integers:
    m1 = smallest integer with m1^3 >= N, m2 = smallest with m1*m2^2 >= N,
    m3 = ceil(N / (m1*m2))."""
    if N < 1:
        raise ValueError("N must be positive")
    m1 = max(1, int(round(N ** (1.0 / 3.0))) - 2)
    while m1 ** 3 < N:
        m1 += 1
    while m1 > 1 and (m1 - 1) ** 3 >= N:
        m1 -= 1
    m2 = max(1, int(math.isqrt(max(0, N // m1))) - 2)
    while m1 * m2 * m2 < N:
        m2 += 1
    while m2 > 1 and m1 * (m2 - 1) * (m2 - 1) >= N:
        m2 -= 1
    m3 = -(-N // (m1 * m2))
    return (m1, m2, m3)


def bounded_zipf(rng: np.random.Generator, N: int, alpha: float, size: int) -> np.ndarray:
    """Ranks k in 1..N with P(k) proportional to k^-alpha, by inverse CDF."""
    k = np.arange(1, N + 1, dtype=np.float64)
    w = k ** (-alpha)
    del k
    cdf = np.cumsum(w)
    del w
    cdf /= cdf[-1]
    u = rng.random(size)
    r = np.searchsorted(cdf, u, side="right") + 1
    np.minimum(r, N, out=r)
    return r.astype(np.int64)


def _core_std(R: int, nk: int) -> float:
    return float((R * nk) ** -0.25)


def _draw_cores(rng, tables: Sequence[Table], std_rule):
    """Draw G1, G2, G3 for each table in order (per table: G1, G2, G3)."""
    g1s, g2s, g3s, goff = [], [], [], []
    o1 = o2 = o3 = 0
    for t in tables:
        m1, m2, m3 = t.m
        n1, n2, n3 = t.n
        R = t.rank
        s1, s2, s3 = std_rule(t)
        a = rng.normal(0.0, s1, (m1, n1, R)).astype(np.float32)
        b = rng.normal(0.0, s2, (m2, R, n2, R)).astype(np.float32)
        c = rng.normal(0.0, s3, (m3, R, n3)).astype(np.float32)
        g1s.append(a.ravel()); g2s.append(b.ravel()); g3s.append(c.ravel())
        goff.append((o1, o2, o3))
        o1 += a.size; o2 += b.size; o3 += c.size
    return (np.concatenate(g1s), np.concatenate(g2s), np.concatenate(g3s),
            np.array(goff, dtype=np.int64))


def _scaled_std(t: Table):
    return (_core_std(t.rank, t.n[0]), _core_std(t.rank, t.n[1]), _core_std(t.rank, t.n[2]))


def _offsets_from_lens(lens: np.ndarray) -> np.ndarray:
    off = np.zeros(lens.size + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    return off


CONFIGS = ("tiny", "table1m", "skew11m", "multi26", "train11m")


def make(name: str, seed: int = 0, batch: Optional[int] = None,
         permuted: bool = False, tables: Optional[int] = None,
         max_rows: Optional[int] = None) -> Problem:
    """Build one of the five synthetic workloads.

    batch    overrides B (bags per table) for smaller parity cases; the draws
             keep their order, so a smaller batch is a different sample.
    permuted applies a random row permutation to skew11m / train11m indices
             (a sensitivity variant; drawn after the indices).
    tables   (multi26 only) keep the first `tables` tables.
    max_rows (multi26 only) cap each table's N, for small parity cases.
    """
    rng = np.random.default_rng(seed)
    if name == "tiny":
        t = Table(1000, (10, 10, 10), (2, 2, 4), 4)
        g1, g2, g3, goff = _draw_cores(rng, [t], lambda _t: (0.1, 0.1, 0.1))
        B = 256 if batch is None else batch
        idx = rng.integers(0, 1000, B).astype(np.int64)
        off = np.arange(B + 1, dtype=np.int64)
        return Problem(name, [t], B, g1, g2, g3, goff, idx, off)

    if name == "table1m":
        t = Table(1_000_000, (100, 100, 100), (4, 4, 4), 16)
        g1, g2, g3, goff = _draw_cores(rng, [t], _scaled_std)
        B = 4096 if batch is None else batch
        k = bounded_zipf(rng, t.num_rows, 1.05, B)
        perm = rng.permutation(t.num_rows).astype(np.int64)
        idx = perm[k - 1]
        off = np.arange(B + 1, dtype=np.int64)
        return Problem(name, [t], B, g1, g2, g3, goff, idx, off)

    if name in ("skew11m", "train11m"):
        t = Table(11_000_000, (200, 220, 250), (4, 8, 4), 32)
        g1, g2, g3, goff = _draw_cores(rng, [t], _scaled_std)
        B = 32768 if batch is None else batch
        lens = np.clip(rng.poisson(20, B), 1, 100).astype(np.int64)
        L = int(lens.sum())
        idx = bounded_zipf(rng, t.num_rows, 1.1, L) - 1
        if permuted:
            perm = rng.permutation(t.num_rows).astype(np.int64)
            idx = perm[idx]
        off = _offsets_from_lens(lens)
        p = Problem(name, [t], B, g1, g2, g3, goff, idx, off)
        if name == "train11m":
            p.grad_out = rng.standard_normal((B, t.dim), dtype=np.float32)
            p.lr = 0.01
        return p

    if name == "multi26":
        T = 26
        Ns = np.rint(np.exp(rng.uniform(math.log(1e3), math.log(4e7), T))).astype(np.int64)
        alphas = rng.uniform(0.8, 1.2, T)
        ntab = T if tables is None else tables
        B = 32768 if batch is None else batch
        tabs: List[Table] = []
        g1s, g2s, g3s, goffs, idxs, lens_all = [], [], [], [], [], []
        o1 = o2 = o3 = 0
        for ti in range(ntab):
            N = int(Ns[ti])
            if max_rows is not None:
                N = min(N, max_rows)
            t = Table(N, near_equal_radices(N), (4, 4, 4), 32)
            tabs.append(t)
            a, b, c, _ = _draw_cores(rng, [t], _scaled_std)
            g1s.append(a); g2s.append(b); g3s.append(c)
            goffs.append((o1, o2, o3))
            o1 += a.size; o2 += b.size; o3 += c.size
            lens = rng.poisson(10, B).astype(np.int64)
            L = int(lens.sum())
            idxs.append(bounded_zipf(rng, N, float(alphas[ti]), L) - 1)
            lens_all.append(lens)
        return Problem(name, tabs, B, np.concatenate(g1s), np.concatenate(g2s),
                       np.concatenate(g3s), np.array(goffs, dtype=np.int64),
                       np.concatenate(idxs), _offsets_from_lens(np.concatenate(lens_all)))

    raise ValueError(f"unknown workload {name!r}; expected one of {CONFIGS}")


def make_custom(tables: Sequence[Table], lens: Sequence[int] | np.ndarray, seed: int = 0,
                std: Optional[float] = None, zipf_alpha: Optional[float] = None,
                with_grad: bool = False, lr: float = 0.01) -> Problem:
    """Small arbitrary problem for property tests: given tables and per-bag
    lengths (length T*B, table-major), draw cores and uniform (or Zipf)
    indices. Every table gets B = len(lens) // T bags."""
    rng = np.random.default_rng(seed)
    T = len(tables)
    lens = np.asarray(lens, dtype=np.int64)
    if lens.size % T:
        raise ValueError("len(lens) must be a multiple of the table count")
    B = lens.size // T
    rule = (lambda _t: (std, std, std)) if std is not None else _scaled_std
    g1, g2, g3, goff = _draw_cores(rng, tables, rule)
    idxs = []
    for ti, t in enumerate(tables):
        Lt = int(lens[ti * B:(ti + 1) * B].sum())
        if zipf_alpha is None:
            idxs.append(rng.integers(0, t.num_rows, Lt).astype(np.int64))
        else:
            idxs.append(bounded_zipf(rng, t.num_rows, zipf_alpha, Lt) - 1)
    idx = np.concatenate(idxs) if idxs else np.zeros(0, np.int64)
    p = Problem("custom", list(tables), B, g1, g2, g3, goff, idx, _offsets_from_lens(lens))
    if with_grad:
        p.grad_out = rng.standard_normal((T * B, tables[0].dim), dtype=np.float32)
        p.lr = lr
    return p
