"""Pins of the forward oracle against mathematics (CPU only).

A plausible slip in the oracle (a dropped term, a wrong index or sign, a
transposed core) breaks at least one of: the brute-force table built by the
other contraction order, the hand-worked example, the rank-1 Kronecker form,
gauge invariance, or linearity in each core.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as wl
from tests import ttref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_2x1x2.json")


def _golden_problem():
    g = json.load(open(GOLDEN))
    t = wl.Table(g["table"]["num_rows"], tuple(g["table"]["m"]), tuple(g["table"]["n"]),
                 g["table"]["rank"])
    p = wl.Problem("golden", [t], g["batch"],
                   np.array(g["g1"], np.float32).ravel(), np.array(g["g2"], np.float32).ravel(),
                   np.array(g["g3"], np.float32).ravel(), np.zeros((1, 3), np.int64),
                   np.array(g["indices"], np.int64), np.array(g["offsets"], np.int64),
                   grad_out=np.array(g["grad_out"], np.float32), lr=g["lr"])
    return g, p


def test_hand_worked_rows_and_bags():
    g, p = _golden_problem()
    rows = oracle.forward(p.tables, p.g1, p.g2, p.g3, p.goff, np.arange(4), np.arange(5), 4)
    np.testing.assert_array_equal(rows, np.array(g["rows"], np.float64))
    np.testing.assert_array_equal(oracle.forward_problem(p), np.array(g["out"], np.float64))


def test_tiny_against_materialised_table():
    """The 1,000 x 16 tiny table: every one of the 256 one-lookup bags equals
    the row of the fully materialised table."""
    p = wl.make("tiny")
    W = ttref.materialise(p.tables[0], p.g1, p.g2, p.g3, p.goff[0])
    assert W.shape == (1000, 16)
    out = oracle.forward_problem(p)
    np.testing.assert_allclose(out, W[p.indices], rtol=1e-12, atol=1e-14)
    # every row of the table, one lookup per bag
    allrows = oracle.forward(p.tables, p.g1, p.g2, p.g3, p.goff, np.arange(1000),
                             np.arange(1001), 1000)
    np.testing.assert_allclose(allrows, W, rtol=1e-12, atol=1e-14)


_NS = [(1, 1, 4), (1, 2, 2), (2, 2, 1), (4, 1, 1), (2, 1, 2), (1, 4, 1)]


@st.composite
def small_problems(draw, with_grad=False):
    T = draw(st.integers(1, 3))
    tabs = []
    for _ in range(T):
        m = tuple(draw(st.integers(1, 4)) for _ in range(3))
        N = draw(st.integers(1, m[0] * m[1] * m[2]))
        n = draw(st.sampled_from(_NS))
        R = draw(st.integers(1, 4))
        tabs.append(wl.Table(N, m, n, R))
    B = draw(st.integers(0, 4))
    lens = np.array([draw(st.integers(0, 4)) for _ in range(T * B)], dtype=np.int64)
    seed = draw(st.integers(0, 2**31 - 1))
    return wl.make_custom(tabs, lens, seed=seed, std=1.0, with_grad=with_grad)


@settings(max_examples=60, deadline=None)
@given(small_problems())
def test_random_small_against_bruteforce(p):
    ref = ttref.pooled_bruteforce(p)
    out = oracle.forward_problem(p)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11)


def test_rank1_kronecker_closed_form():
    """R = 1: the row is kron(kron(G1[i1][:,0], G2[i2][0,:,0]), G3[i3][0,:])."""
    rng = np.random.default_rng(7)
    t = wl.Table(5 * 3 * 4, (5, 3, 4), (2, 3, 2), 1)
    g1 = rng.standard_normal(5 * 2).astype(np.float32)
    g2 = rng.standard_normal(3 * 3).astype(np.float32)
    g3 = rng.standard_normal(4 * 2).astype(np.float32)
    idx = np.arange(60, dtype=np.int64)
    out = oracle.forward([t], g1, g2, g3, np.zeros((1, 3), np.int64), idx, np.arange(61), 60)
    for x in range(60):
        i1, rem = divmod(x, 12)
        i2, i3 = divmod(rem, 4)
        want = np.kron(np.kron(g1.reshape(5, 2)[i1].astype(np.float64),
                               g2.reshape(3, 3)[i2].astype(np.float64)),
                       g3.reshape(4, 2)[i3].astype(np.float64))
        np.testing.assert_allclose(out[x], want, rtol=1e-12, atol=1e-14)


def _orth(rng, R):
    q, r = np.linalg.qr(rng.standard_normal((R, R)))
    return q * np.sign(np.diag(r))


def test_gauge_invariance():
    """Inserting Q Q^T on either internal rank bond leaves every row unchanged."""
    p = wl.make("tiny")
    t = p.tables[0]
    rng = np.random.default_rng(3)
    R = t.rank
    A, B, C = ttref.core_views(t, p.g1, p.g2, p.g3, p.goff[0])
    base = oracle.forward(p.tables, p.g1, p.g2, p.g3, p.goff, np.arange(1000),
                          np.arange(1001), 1000)
    Q = _orth(rng, R)
    # bond r1: G1 <- G1 Q, G2 <- Q^T G2 (on the r1 index)
    A2 = np.einsum("aix,xy->aiy", A, Q)
    B2 = np.einsum("xy,bxjs->byjs", Q, B)
    # bond r2: G2 <- G2 Q (on r2), G3 <- Q^T G3
    Q2 = _orth(rng, R)
    B3 = np.einsum("byjs,st->byjt", B2, Q2)
    C3 = np.einsum("st,csk->ctk", Q2, C)
    # The oracle reads fp32 cores, so compare against the same rotated fp32 cores
    # through the independent materialisation instead of against `base` directly.
    f32 = lambda x: x.astype(np.float32).ravel()
    rot = oracle.forward(p.tables, f32(A2), f32(B3), f32(C3), p.goff, np.arange(1000),
                         np.arange(1001), 1000)
    W = ttref.materialise(t, f32(A2), f32(B3), f32(C3), p.goff[0])
    np.testing.assert_allclose(rot, W, rtol=1e-10, atol=1e-12)
    # and the rotation itself is exact up to fp32 rounding of the rotated cores
    np.testing.assert_allclose(rot, base, rtol=1e-5, atol=1e-6)


def test_linearity_in_each_core_and_pooling_additivity():
    p = wl.make("tiny", batch=64)
    rng = np.random.default_rng(11)
    f = lambda a, b, c: oracle.forward(p.tables, a, b, c, p.goff, p.indices, p.offsets, p.batch)
    base = f(p.g1, p.g2, p.g3)
    for k in range(3):
        cores = [p.g1, p.g2, p.g3]
        V = rng.integers(-3, 4, cores[k].size).astype(np.float32)
        mix = list(cores); mix[k] = (cores[k] + np.float32(2.0) * V).astype(np.float32)
        only = list(cores); only[k] = V
        # the mixed core is rounded to fp32, hence the loose tolerance
        np.testing.assert_allclose(f(*mix), base + 2.0 * f(*only), rtol=1e-5, atol=1e-5)
    # pooling additivity: one bag holding all lookups equals the sum of the rows
    allbag = oracle.forward(p.tables, p.g1, p.g2, p.g3, p.goff, p.indices,
                            np.array([0, p.L]), 1)
    np.testing.assert_allclose(allbag[0], base.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_empty_bags_and_errors():
    t = wl.Table(30, (2, 3, 5), (1, 2, 2), 2)
    p = wl.make_custom([t], np.array([0, 3, 0, 2]), seed=1)
    out = oracle.forward_problem(p)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.any(out[1] != 0)
    bad = p.indices.copy(); bad[0] = 30
    with pytest.raises(oracle.OracleError):
        oracle.forward(p.tables, p.g1, p.g2, p.g3, p.goff, bad, p.offsets, p.batch)
    bad[0] = -1
    with pytest.raises(oracle.OracleError):
        oracle.forward(p.tables, p.g1, p.g2, p.g3, p.goff, bad, p.offsets, p.batch)
    off = p.offsets.copy(); off[2] = off[1] - 1
    with pytest.raises(oracle.OracleError):
        oracle.forward(p.tables, p.g1, p.g2, p.g3, p.goff, p.indices, off, p.batch)


def test_sampled_bags_match_full():
    p = wl.make("skew11m", batch=48)
    full = oracle.forward_problem(p)
    bags = np.array([47, 0, 13, 13, 30])
    np.testing.assert_array_equal(oracle.forward_problem(p, bags=bags), full[bags])
