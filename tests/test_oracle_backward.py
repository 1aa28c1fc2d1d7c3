"""Pins of the backward and SGD oracles (CPU only).

The forward is linear in each core, so for any V shaped like core k,
<dL/dG_k, V> = <grad_out, F(cores with G_k replaced by V)> exactly. That
identity uses only the (separately pinned) forward oracle. The hand-worked
example and a chain rule through the materialised table pin it further.
"""
import json
import os

import numpy as np
from hypothesis import given, settings

import oracle
import workloads as wl
from tests import ttref
from tests.test_oracle_forward import _golden_problem, small_problems


def test_hand_worked_gradients_and_sgd():
    g, p = _golden_problem()
    d1, d2, d3 = oracle.backward_problem(p)
    np.testing.assert_array_equal(d1, np.array(g["dg1"], np.float64).ravel())
    np.testing.assert_array_equal(d2, np.array(g["dg2"], np.float64).ravel())
    np.testing.assert_array_equal(d3, np.array(g["dg3"], np.float64).ravel())
    np.testing.assert_array_equal(oracle.sgd(p.g3, d3, g["lr"]),
                                  np.array(g["sgd_g3"], np.float64).ravel())
    out = oracle.forward_problem(p)
    assert float(np.sum(out * p.grad_out)) == g["loss"]


def _adjoint_check(p, rng, rtol=1e-10):
    d = oracle.backward_problem(p)
    cores = [p.g1, p.g2, p.g3]
    for k in range(3):
        V = rng.standard_normal(cores[k].size).astype(np.float32)
        sub = list(cores); sub[k] = V
        Fv = oracle.forward(p.tables, *sub, p.goff, p.indices, p.offsets, p.batch)
        lhs = float(np.dot(d[k], V.astype(np.float64)))
        rhs = float(np.sum(Fv * p.grad_out.astype(np.float64)))
        scale = float(np.dot(np.abs(d[k]), np.abs(V))) + 1e-30
        assert abs(lhs - rhs) <= rtol * scale, (k, lhs, rhs)


def test_adjoint_identity_skew_shapes():
    p = wl.make("train11m", batch=24)
    _adjoint_check(p, np.random.default_rng(5))


def test_adjoint_identity_multitable():
    p = wl.make("multi26", batch=16, tables=3, max_rows=5000)
    p.grad_out = np.random.default_rng(9).standard_normal((p.T * p.batch, p.dim)).astype(np.float32)
    _adjoint_check(p, np.random.default_rng(6))


@settings(max_examples=40, deadline=None)
@given(small_problems(with_grad=True))
def test_random_small_against_chain_rule(p):
    ref = ttref.grads_bruteforce(p)
    got = oracle.backward_problem(p)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


def test_rank1_gradient_closed_form():
    """R = 1, one lookup: dG3[i3][0][j3] = sum_{j1,j2} a[j1] b[j2] g[j1,j2,j3]."""
    rng = np.random.default_rng(2)
    t = wl.Table(2 * 2 * 3, (2, 2, 3), (2, 3, 2), 1)
    g1 = rng.standard_normal(2 * 2).astype(np.float32)
    g2 = rng.standard_normal(2 * 3).astype(np.float32)
    g3 = rng.standard_normal(3 * 2).astype(np.float32)
    go = rng.standard_normal((1, 12)).astype(np.float32)
    idx = np.array([7], np.int64)             # i1=1, i2=0, i3=1
    d1, d2, d3 = oracle.backward([t], g1, g2, g3, np.zeros((1, 3), np.int64), idx,
                                 np.array([0, 1]), 1, go)
    a, b, c = g1.reshape(2, 2)[1], g2.reshape(2, 3)[0], g3.reshape(3, 2)[1]
    G = go.reshape(2, 3, 2).astype(np.float64)
    np.testing.assert_allclose(d3.reshape(3, 2)[1], np.einsum("i,j,ijk->k", a, b, G), rtol=1e-12)
    np.testing.assert_allclose(d2.reshape(2, 3)[0], np.einsum("i,k,ijk->j", a, c, G), rtol=1e-12)
    np.testing.assert_allclose(d1.reshape(2, 2)[1], np.einsum("j,k,ijk->i", b, c, G), rtol=1e-12)
    # untouched slices are exactly zero
    assert np.all(d3.reshape(3, 2)[[0, 2]] == 0) and np.all(d1.reshape(2, 2)[0] == 0)


def test_mask_partition_sums_to_full():
    p = wl.make("train11m", batch=16)
    full = oracle.backward_problem(p)
    mask = (np.arange(p.L) % 3 == 0).astype(np.uint8)
    a = oracle.backward_problem(p, mask=mask)
    b = oracle.backward_problem(p, mask=1 - mask)
    for f, x, y in zip(full, a, b):
        np.testing.assert_allclose(x + y, f, rtol=1e-12, atol=1e-12)


def test_hot_slice_fixture_inputs_current():
    """The stored hot-slice gradients (tests/golden/train11m_hot_slices.npz,
    written by the oracle) belong to the inputs the generator draws today."""
    import workloads as wl
    from tests.golden.make_train11m_hot_slices import OUT, fingerprint
    g = np.load(OUT)
    p = wl.make("train11m")
    assert str(g["fingerprint"]) == fingerprint(p)
    t = p.tables[0]
    R, (n1, n2, n3) = t.rank, t.n
    assert g["dg1_i1_0"].shape == (n1 * R,)
    assert g["dg2_i2_0"].shape == (R * n2 * R,)
    assert g["dg3_i3_0"].shape == (R * n3,)


def test_shared_core_is_the_sum_of_its_tables():
    """Two tables reading one G3 (same offset): the gradient of the shared G3
    is the sum of what each table alone gives it, and G1, G2 split by table.
    (The per-slice accumulation runs in parallel; slices of tables that share
    elements must not, and this is the case where they would collide.)"""
    t1 = wl.Table(4 * 5 * 300, (4, 5, 300), (4, 8, 4), 8)
    t2 = wl.Table(3 * 6 * 300, (3, 6, 300), (4, 8, 4), 8)
    p = wl.make_custom([t1, t2], np.full(2 * 60, 7), seed=7, zipf_alpha=1.1, with_grad=True)
    g3 = p.g3[:300 * 8 * 4].copy()
    goff = p.goff.copy()
    goff[1, 2] = 0
    shared = wl.Problem("shared", p.tables, p.batch, p.g1, p.g2, g3, goff, p.indices, p.offsets,
                        p.grad_out, p.lr)
    B, L1 = p.batch, int(p.offsets[p.batch])
    parts = []
    for t, (lo, hi) in enumerate([(0, L1), (L1, p.L)]):
        off = p.offsets[t * B:(t + 1) * B + 1] - p.offsets[t * B]
        q = wl.Problem("one", [p.tables[t]], B, p.g1, p.g2, g3, goff[t:t + 1], p.indices[lo:hi],
                       off, p.grad_out[t * B:(t + 1) * B], p.lr)
        parts.append(oracle.backward_problem(q))
    for _ in range(5):   # a collision between threads shows up only now and then
        d = oracle.backward_problem(shared)
        for k in range(3):
            np.testing.assert_allclose(d[k], parts[0][k] + parts[1][k], rtol=1e-12, atol=1e-12)
