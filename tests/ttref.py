"""Independent NumPy constructions used to pin the oracle (CPU only).

These are not the oracle: they compute the same quantities by other routes
(materialising the whole table by contracting G2 with G3 first, the rank-1
Kronecker form, the chain rule through the materialised table), so that an
error in the oracle's own loops would show up as a disagreement.
"""
from __future__ import annotations

import numpy as np


def core_views(t, g1, g2, g3, goff):
    """float64 views [m1][n1][R], [m2][R][n2][R], [m3][R][n3] of one table."""
    m1, m2, m3 = t.m
    n1, n2, n3 = t.n
    R = t.rank
    o1, o2, o3 = (int(x) for x in goff)
    A = np.asarray(g1[o1:o1 + m1 * n1 * R], np.float64).reshape(m1, n1, R)
    B = np.asarray(g2[o2:o2 + m2 * R * n2 * R], np.float64).reshape(m2, R, n2, R)
    C = np.asarray(g3[o3:o3 + m3 * R * n3], np.float64).reshape(m3, R, n3)
    return A, B, C


def materialise(t, g1, g2, g3, goff):
    """Full table W [m1*m2*m3][D], rows (i1*m2+i2)*m3+i3, cols (j1*n2+j2)*n3+j3.
    Contracts G2 with G3 first (the opposite order to the oracle's chain)."""
    A, B, C = core_views(t, g1, g2, g3, goff)
    S = np.einsum("bxjs,csk->bcxjk", B, C)          # [m2][m3][r1][n2][n3]
    W = np.einsum("aix,bcxjk->abcijk", A, S)        # [m1][m2][m3][n1][n2][n3]
    m1, m2, m3 = t.m
    return W.reshape(m1 * m2 * m3, t.dim)


def pooled_bruteforce(p):
    """out[q] = sum of materialised rows of bag q, per table."""
    D = p.tables[0].dim
    out = np.zeros((p.T * p.batch, D))
    for ti, t in enumerate(p.tables):
        W = materialise(t, p.g1, p.g2, p.g3, p.goff[ti])
        for b in range(p.batch):
            q = ti * p.batch + b
            for l in range(p.offsets[q], p.offsets[q + 1]):
                out[q] += W[p.indices[l]]
    return out


def grads_bruteforce(p):
    """Core gradients by the chain rule through the materialised table:
    dW = sum_l e_{idx_l} g_l^T, then contract dW with the two other cores."""
    d1 = np.zeros(p.g1.size); d2 = np.zeros(p.g2.size); d3 = np.zeros(p.g3.size)
    for ti, t in enumerate(p.tables):
        m1, m2, m3 = t.m
        n1, n2, n3 = t.n
        R = t.rank
        A, B, C = core_views(t, p.g1, p.g2, p.g3, p.goff[ti])
        dW = np.zeros((m1 * m2 * m3, t.dim))
        for b in range(p.batch):
            q = ti * p.batch + b
            for l in range(p.offsets[q], p.offsets[q + 1]):
                dW[p.indices[l]] += p.grad_out[q]
        dW = dW.reshape(m1, m2, m3, n1, n2, n3)
        dA = np.einsum("abcijk,bxjs,csk->aix", dW, B, C)
        dB = np.einsum("abcijk,aix,csk->bxjs", dW, A, C)
        dC = np.einsum("abcijk,aix,bxjs->csk", dW, A, B)
        o1, o2, o3 = (int(x) for x in p.goff[ti])
        d1[o1:o1 + dA.size] = dA.ravel()
        d2[o2:o2 + dB.size] = dB.ravel()
        d3[o3:o3 + dC.size] = dC.ravel()
    return d1, d2, d3


def plan_bruteforce(radices, num_rows, B, indices, offsets, chunk):
    """Planner tables by plain Python: digits by repeated division, order by
    Python's sorted() on (key, i3, l) tuples, groups and chunks by walking."""
    L = len(indices)
    bag = []
    for q in range(len(offsets) - 1):
        bag += [q] * int(offsets[q + 1] - offsets[q])
    base = [0]
    for (m1, m2, _m3) in radices:
        base.append(base[-1] + m1 * m2)
    i1s, i2s, i3s, keys = [], [], [], []
    for l in range(L):
        t = bag[l] // B
        m1, m2, m3 = radices[t]
        x = int(indices[l])
        assert 0 <= x < num_rows[t]
        i3 = x % m3
        x //= m3
        i2 = x % m2
        i1 = x // m2
        i1s.append(i1); i2s.append(i2); i3s.append(i3)
        keys.append(base[t] + i2 * m1 + i1)
    order = [l for (_k, _i, l) in sorted((keys[l], i3s[l], l) for l in range(L))]
    gk, gs = [], []
    for s, l in enumerate(order):
        if s == 0 or keys[l] != keys[order[s - 1]]:
            gk.append(keys[l]); gs.append(s)
    gs.append(L)
    cg, cb, ce = [], [], []
    for g in range(len(gk)):
        s = gs[g]
        while s < gs[g + 1]:
            e = min(s + chunk, gs[g + 1])
            cg.append(g); cb.append(s); ce.append(e)
            s = e
    return {
        "bag_of": bag, "i1": i1s, "i2": i2s, "i3": i3s, "key": keys, "perm": order,
        "sorted_i3": [i3s[l] for l in order], "sorted_bag": [bag[l] for l in order],
        "group_key": gk, "group_start": gs, "chunk_group": cg, "chunk_begin": cb,
        "chunk_end": ce,
    }
