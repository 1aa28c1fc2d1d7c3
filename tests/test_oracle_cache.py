"""Pins of the oracle's hot-row cache (TT-Rec abstract: caching strategies for
the lookups; TT-Rec news article, method: a cache structure for the skewed
feature distribution). Each pin rests on something other than the cache
code's own arithmetic: the plain forward and backward oracles (themselves
pinned), linearity, and brute force on tiny inputs."""
import numpy as np

import oracle
import workloads as wl


def _problem(seed=0, tables=None, lens=None):
    tables = tables or [wl.Table(20 * 12 * 30, (20, 12, 30), (2, 2, 4), 4)]
    lens = np.random.default_rng(seed).poisson(6, 40 * len(tables)) if lens is None else lens
    return wl.make_custom(tables, lens, seed=seed, zipf_alpha=1.1, with_grad=True)


def _hot(p, k, seed=1):
    """The k most frequent (table, row) pairs of the batch."""
    bag = np.repeat(np.arange(p.T * p.batch), np.diff(p.offsets))
    key = (bag // p.batch) * (1 << 40) + p.indices
    u, c = np.unique(key, return_counts=True)
    top = u[np.argsort(-c, kind="stable")[:k]]
    return (top >> 40).astype(np.int64), (top & ((1 << 40) - 1)).astype(np.int64)


def test_empty_hot_set_changes_nothing():
    p = _problem()
    e = np.zeros(0, np.int64)
    W = np.zeros((0, p.dim), np.float32)
    np.testing.assert_array_equal(oracle.forward_cached(p, e, e, W), oracle.forward_problem(p))
    d = oracle.backward_cached(p, e, e, 0)
    for a, b in zip(d[:3], oracle.backward_problem(p)):
        np.testing.assert_array_equal(a, b)
    assert d[3].shape == (0, p.dim)


def test_hot_rows_holding_their_tt_values_reproduce_the_forward():
    for tables in (None, [wl.Table(900, (9, 10, 10), (2, 2, 4), 3), wl.Table(500, (5, 10, 10), (2, 2, 4), 5)]):
        p = _problem(seed=2, tables=tables)
        ht, hr = _hot(p, 7)
        W = oracle.materialise_rows(p, ht, hr)
        got = oracle.forward_cached(p, ht, hr, W)
        np.testing.assert_allclose(got, oracle.forward_problem(p), rtol=1e-12, atol=1e-12)
        assert (oracle.cache_slots(p, ht, hr) >= 0).sum() > 0


def test_materialised_rows_by_brute_force():
    """Row r of a table is G1[i1] G2[i2] G3[i3] with i1 most significant."""
    p = _problem(seed=3)
    t = p.tables[0]
    ht, hr = np.zeros(5, np.int64), np.array([0, 1, 37, 7199, 4000], np.int64)
    W = oracle.materialise_rows(p, ht, hr)
    R, (n1, n2, n3), (m1, m2, m3) = t.rank, t.n, t.m
    G1 = p.g1.reshape(m1, n1, R).astype(np.float64)
    G2 = p.g2.reshape(m2, R, n2, R).astype(np.float64)
    G3 = p.g3.reshape(m3, R, n3).astype(np.float64)
    for s, r in enumerate(hr):
        i1, rest = divmod(int(r), m2 * m3)
        i2, i3 = divmod(rest, m3)
        row = np.einsum("ar,rbs,sc->abc", G1[i1], G2[i2], G3[i3]).reshape(-1)
        np.testing.assert_allclose(W[s], row, rtol=1e-12, atol=1e-12)


def test_dw_adjoint_identity():
    """out is affine in W: <dW, V> = <grad_out, out(W=V) - out(W=0)>."""
    p = _problem(seed=4)
    ht, hr = _hot(p, 6)
    V = np.random.default_rng(5).standard_normal((6, p.dim))
    dW = oracle.backward_cached(p, ht, hr, 6)[3]
    lhs = float(np.sum(dW * V))
    diff = oracle.forward_cached(p, ht, hr, V) - oracle.forward_cached(p, ht, hr, np.zeros_like(V))
    rhs = float(np.sum(np.asarray(p.grad_out, np.float64) * diff))
    assert abs(lhs - rhs) <= 1e-10 * (1 + abs(rhs))


def test_core_gradients_partition_over_hot_and_cold_lookups():
    p = _problem(seed=6, tables=[wl.Table(900, (9, 10, 10), (2, 2, 4), 3), wl.Table(500, (5, 10, 10), (2, 2, 4), 5)])
    ht, hr = _hot(p, 9)
    cold = oracle.backward_cached(p, ht, hr, 9)[:3]
    hot = oracle.backward_problem(p, mask=(oracle.cache_slots(p, ht, hr) >= 0).astype(np.uint8))
    for c, h, a in zip(cold, hot, oracle.backward_problem(p)):
        np.testing.assert_allclose(c + h, a, rtol=1e-12, atol=1e-12)


def test_slots_by_brute_force_with_duplicates_and_tables():
    """A pair listed twice is served by its first slot; the same row number
    in another table is another pair."""
    p = _problem(seed=7, tables=[wl.Table(900, (9, 10, 10), (2, 2, 4), 3), wl.Table(900, (9, 10, 10), (2, 2, 4), 3)])
    r0 = int(p.indices[0])
    ht = np.array([0, 1, 0, 0], np.int64)
    hr = np.array([r0, r0, r0, (r0 + 1) % 900], np.int64)
    slot = oracle.cache_slots(p, ht, hr)
    bag = np.repeat(np.arange(p.T * p.batch), np.diff(p.offsets))
    for l in range(p.L):
        t, r = bag[l] // p.batch, int(p.indices[l])
        want = -1
        for s in range(4):
            if ht[s] == t and hr[s] == r:
                want = s
                break
        assert slot[l] == want
    dW = oracle.backward_cached(p, ht, hr, 4)[3]
    assert not dW[2].any()   # the duplicate's slot takes no lookups
