"""Pins of the planner oracle (CPU only): digit identity over every row,
the hand-worked plan, a pure-Python brute-force planner, and the partition
invariants of the group and chunk tables."""
import json

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import planner
import workloads as wl
from tests import ttref
from tests.test_oracle_forward import GOLDEN


@pytest.mark.parametrize("m,N", [((10, 10, 10), 1000), ((3, 5, 7), 100), ((1, 1, 9), 9),
                                 ((200, 220, 250), 11_000_000)])
def test_split_digit_identity(m, N):
    idx = np.arange(N, dtype=np.int64) if N <= 200_000 else \
        np.random.default_rng(0).integers(0, N, 200_000)
    p = planner.plan([m], [N], idx.size, idx, np.arange(idx.size + 1), 7)
    i1, i2, i3 = (p[k].astype(np.int64) for k in ("i1", "i2", "i3"))
    assert np.all((0 <= i1) & (i1 < m[0]) & (0 <= i2) & (i2 < m[1]) & (0 <= i3) & (i3 < m[2]))
    np.testing.assert_array_equal((i1 * m[1] + i2) * m[2] + i3, idx)
    np.testing.assert_array_equal(p["key"].astype(np.int64), i2 * m[0] + i1)


def test_hand_worked_plan():
    g = json.load(open(GOLDEN))
    p = planner.plan([tuple(g["table"]["m"])], [g["table"]["num_rows"]], g["batch"],
                     np.array(g["indices"]), np.array(g["offsets"]), g["plan_chunk"])
    for k, v in g["plan"].items():
        np.testing.assert_array_equal(p[k], np.array(v, np.int32), err_msg=k)


@st.composite
def plan_inputs(draw):
    T = draw(st.integers(1, 3))
    radices, Ns = [], []
    for _ in range(T):
        m = tuple(draw(st.integers(1, 5)) for _ in range(3))
        radices.append(m)
        Ns.append(draw(st.integers(1, m[0] * m[1] * m[2])))
    B = draw(st.integers(0, 6))
    lens = [draw(st.integers(0, 5)) for _ in range(T * B)]
    idx = []
    for q, n in enumerate(lens):
        t = q // B
        idx += [draw(st.integers(0, Ns[t] - 1)) for _ in range(n)]
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    chunk = draw(st.integers(1, 4))
    return radices, Ns, B, np.array(idx, np.int64), off, chunk


@settings(max_examples=200, deadline=None)
@given(plan_inputs())
def test_against_bruteforce(inp):
    radices, Ns, B, idx, off, chunk = inp
    got = planner.plan(radices, Ns, B, idx, off, chunk)
    ref = ttref.plan_bruteforce(radices, Ns, B, idx, off, chunk)
    for k, v in ref.items():
        np.testing.assert_array_equal(got[k], np.array(v, np.int64).astype(np.int32), err_msg=k)


def check_invariants(p, L, chunk):
    perm = p["perm"].astype(np.int64)
    assert np.array_equal(np.sort(perm), np.arange(L))
    skey = p["key"][perm].astype(np.int64)
    si3 = p["i3"][perm].astype(np.int64)
    assert np.all(np.diff(skey) >= 0)
    same_key = np.diff(skey) == 0
    assert np.all(np.diff(si3)[same_key] >= 0)            # i3 ascending inside a group
    ties = same_key & (np.diff(si3) == 0)
    assert np.all(np.diff(perm)[ties] > 0)               # stable on equal (key, i3)
    gs = p["group_start"].astype(np.int64)
    assert gs[0] == 0 and gs[-1] == L and np.all(np.diff(gs) > 0)
    assert np.all(skey[gs[:-1]] == p["group_key"])
    assert np.all(np.diff(p["group_key"]) > 0)
    cb, ce, cg = (p[k].astype(np.int64) for k in ("chunk_begin", "chunk_end", "chunk_group"))
    assert np.all(ce - cb >= 1) and np.all(ce - cb <= chunk)
    assert np.all(cb[1:] == ce[:-1]) and (L == 0 or (cb[0] == 0 and ce[-1] == L))
    assert np.all((gs[cg] <= cb) & (ce <= gs[cg + 1]))    # no chunk spans two groups
    full = (ce - cb) == chunk
    last = ce == gs[cg + 1]
    assert np.all(full | last)                            # only a group's last piece is short
    np.testing.assert_array_equal(p["sorted_i3"], p["i3"][perm])
    np.testing.assert_array_equal(p["sorted_bag"], p["bag_of"][perm])


def test_invariants_skewed_and_multitable():
    p = wl.make("skew11m", batch=2048)
    check_invariants(oracle.plan_problem(p, 256), p.L, 256)
    p = wl.make("multi26", batch=512, tables=5, max_rows=200_000)
    pl = oracle.plan_problem(p, 64)
    check_invariants(pl, p.L, 64)
    # keys of table t lie in [base_t, base_t + m1*m2)
    base = np.concatenate([[0], np.cumsum([t.m[0] * t.m[1] for t in p.tables])])
    t_of = pl["bag_of"] // p.batch
    assert np.all((base[t_of] <= pl["key"]) & (pl["key"] < base[t_of + 1]))


def test_empty_and_errors():
    p = planner.plan([(2, 2, 2)], [8], 3, np.zeros(0, np.int64), np.zeros(4, np.int64), 4)
    assert p["group_start"].tolist() == [0] and p["chunk_begin"].size == 0
    with pytest.raises(planner.PlanError):
        planner.plan([(2, 2, 2)], [7], 1, np.array([7]), np.array([0, 1]), 4)
    with pytest.raises(planner.PlanError):
        planner.plan([(2, 2, 2)], [8], 2, np.array([1, 2]), np.array([0, 2, 1]), 4)
    with pytest.raises(planner.PlanError):
        planner.plan([(2, 2, 2)], [8], 1, np.array([1]), np.array([0, 1]), 0)
