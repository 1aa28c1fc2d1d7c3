"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Planner tables must match bit for bit. Floats must satisfy
|gpu - ref| <= 1e-4 * (1 + |ref|) elementwise, ref being the fp64 oracle.
Every case compares every output element, the full-size workloads included
(the forward of all 32,768 and 851,968 bags; the training step exactly as the
benchmark times it, with every gradient and every updated core element),
except the 26-table backward, which compares sampled slices.
"""
import json

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.test_oracle_forward import GOLDEN

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from tests.gpu_helpers import DevProblem, assert_close, say  # noqa: E402

PLAN_KEYS = ("key", "i3", "bag_of", "perm", "sorted_i3", "sorted_bag", "group_key",
             "group_start", "chunk_group", "chunk_begin", "chunk_end")


def check_plan(dp, label):
    got = dp.plan_tables()
    ref = oracle.plan_problem(dp.p, dp.chunk)
    for k in PLAN_KEYS:
        np.testing.assert_array_equal(got[k], ref[k], err_msg=f"{label}: {k}")
    return got


def run_forward_check(p, label, chunk=256, bags=None):
    say(label, f"L={p.L} bags={p.T * p.batch} chunk={chunk}")
    dp = DevProblem(p, chunk)
    out = dp.forward().cpu().numpy()
    assert dp.plan is not None
    from tensor_train_compressed_amd import tt_emb_get_error
    assert tt_emb_get_error(dp.plan) == 0
    if bags is None:
        ref = oracle.forward_problem(p)
        err = assert_close(out, ref, f"{label} forward")
    else:
        ref = oracle.forward_problem(p, bags=bags)
        err = assert_close(out[bags], ref, f"{label} forward (sampled)")
    say(label, f"max rel err {err:.2e}")
    return dp, out


# ---------------------------------------------------------------------------
# planner

def test_plan_hand_worked():
    g = json.load(open(GOLDEN))
    t = wl.Table(g["table"]["num_rows"], tuple(g["table"]["m"]), tuple(g["table"]["n"]),
                 g["table"]["rank"])
    p = wl.Problem("golden", [t], g["batch"], np.array(g["g1"], np.float32).ravel(),
                   np.array(g["g2"], np.float32).ravel(), np.array(g["g3"], np.float32).ravel(),
                   np.zeros((1, 3), np.int64), np.array(g["indices"], np.int64),
                   np.array(g["offsets"], np.int64), np.array(g["grad_out"], np.float32), g["lr"])
    dp = DevProblem(p, g["plan_chunk"])
    dp.make_plan()
    got = dp.plan_tables()
    for k in PLAN_KEYS:
        np.testing.assert_array_equal(got[k], np.array(g["plan"][k], np.int32), err_msg=k)
    out = dp.forward().cpu().numpy()
    np.testing.assert_allclose(out, np.array(g["out"], np.float64), rtol=0, atol=1e-5)
    d1, d2, d3 = (x.cpu().numpy() for x in dp.backward())
    np.testing.assert_allclose(d1, np.array(g["dg1"], np.float64).ravel(), atol=1e-5)
    np.testing.assert_allclose(d2, np.array(g["dg2"], np.float64).ravel(), atol=1e-5)
    np.testing.assert_allclose(d3, np.array(g["dg3"], np.float64).ravel(), atol=1e-5)


@pytest.mark.parametrize("name,kw,chunk", [
    ("tiny", {}, 256), ("tiny", {}, 1), ("table1m", {}, 256), ("skew11m", {}, 256),
    ("skew11m", {"permuted": True}, 128), ("multi26", {}, 256)])
def test_plan_bit_exact_full_size(name, kw, chunk):
    p = wl.make(name, **kw)
    say("plan", name, kw, f"L={p.L}")
    dp = DevProblem(p, chunk)
    dp.make_plan()
    check_plan(dp, f"{name}{kw}")
    # repeat: identical tables
    first = dp.plan_tables()
    dp.make_plan()
    again = dp.plan_tables()
    for k in PLAN_KEYS:
        np.testing.assert_array_equal(first[k], again[k], err_msg=f"repeat {k}")


def test_plan_edge_cases():
    t = wl.Table(1000, (10, 10, 10), (2, 2, 4), 4)
    cases = {
        "empty bags": wl.make_custom([t], np.array([0, 0, 3, 0, 5, 0]), seed=1),
        "one giant group": wl.make_custom([t], np.full(40, 200), seed=2),
        "all lookups empty": wl.make_custom([t], np.zeros(7, np.int64), seed=3),
    }
    cases["one giant group"].indices[:] = 7          # every lookup -> same (i1, i2)
    cases["empty bags"].indices[-1] = 999            # largest index
    for label, p in cases.items():
        for chunk in (1, 3, 256):
            say("plan edge", label, chunk)
            dp = DevProblem(p, chunk)
            dp.make_plan()
            check_plan(dp, f"{label} chunk={chunk}")


def test_plan_ragged_multitable():
    tabs = [wl.Table(97, (5, 4, 5), (2, 2, 2), 3), wl.Table(1, (1, 1, 1), (1, 8, 1), 2),
            wl.Table(5000, (17, 18, 17), (4, 2, 1), 5)]
    p = wl.make_custom(tabs, np.random.default_rng(0).integers(0, 9, 3 * 700), seed=4)
    for chunk in (1, 7, 64):
        dp = DevProblem(p, chunk)
        dp.make_plan()
        check_plan(dp, f"ragged chunk={chunk}")


def test_plan_many_keys():
    # 2.3M possible prefix keys: more key tiles than one workgroup adds up
    # itself, so the key-tile totals take the device-wide scan
    t = wl.Table(2_300_000, (2300, 1000, 1), (1, 2, 2), 2)
    p = wl.make_custom([t], np.full(64, 40), seed=5)
    for chunk in (1, 64):
        say("plan many keys", chunk)
        dp = DevProblem(p, chunk)
        dp.make_plan()
        check_plan(dp, f"many keys chunk={chunk}")
    run_forward_check(p, "many keys")


def test_device_error_flags():
    from tensor_train_compressed_amd import TT_FLAG_BAD_INDEX, TT_FLAG_BAD_OFFSETS, tt_emb_get_error
    t = wl.Table(1000, (10, 10, 10), (2, 2, 4), 4)
    p = wl.make_custom([t], np.array([2, 3, 1]), seed=5)
    p.indices[3] = 1000
    dp = DevProblem(p)
    dp.make_plan()
    assert tt_emb_get_error(dp.plan) == TT_FLAG_BAD_INDEX
    p = wl.make_custom([t], np.array([2, 3, 1]), seed=5)
    p.indices[0] = -4
    dp = DevProblem(p)
    dp.make_plan()
    assert tt_emb_get_error(dp.plan) == TT_FLAG_BAD_INDEX
    p = wl.make_custom([t], np.array([2, 3, 1]), seed=5)
    p.offsets[1], p.offsets[2] = 4, 3                 # decreasing
    dp = DevProblem(p)
    dp.make_plan()
    assert tt_emb_get_error(dp.plan) & TT_FLAG_BAD_OFFSETS
    dp.forward()                                      # still runs, in bounds
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# forward

def test_forward_tiny_materialised():
    p = wl.make("tiny")
    run_forward_check(p, "tiny")


@pytest.mark.parametrize("chunk", [1, 5, 256])
def test_forward_small_all_bags(chunk):
    run_forward_check(wl.make("skew11m", batch=512), f"skew11m B=512", chunk=chunk)


def test_forward_table1m_full():
    run_forward_check(wl.make("table1m"), "table1m")


def test_forward_multitable_small_all_bags():
    run_forward_check(wl.make("multi26", batch=128), "multi26 B=128")


def test_forward_ragged_shapes():
    tabs = [wl.Table(97, (5, 4, 5), (2, 2, 2), 3), wl.Table(1, (1, 1, 1), (1, 8, 1), 2),
            wl.Table(5000, (17, 18, 17), (4, 2, 1), 5)]
    p = wl.make_custom(tabs, np.random.default_rng(0).integers(0, 9, 3 * 300), seed=4)
    for chunk in (1, 3, 64):
        run_forward_check(p, f"ragged chunk={chunk}", chunk=chunk)


@pytest.mark.parametrize("name,kw", [("skew11m", {}), ("skew11m", {"permuted": True}), ("multi26", {})])
def test_forward_full_size_all_bags(name, kw):
    """The full batches: 32,768 bags of the 11M-row table (unpermuted Zipf,
    and with its rows permuted: far more, smaller prefix groups) and the
    26-table batch (851,968 bags in one launch); every bag."""
    p = wl.make(name, **kw)
    run_forward_check(p, f"{name}{kw} full", chunk=256)


def test_repeat_runs():
    # the forward sums every bag in a fixed order: the same bits on every run;
    # the backward's fp64 accumulation order varies between runs, its fp32
    # result stays within the tolerance of itself
    p = wl.make("train11m")
    dp = DevProblem(p, 256)
    a = dp.forward().cpu().numpy()
    b = dp.forward().cpu().numpy()
    np.testing.assert_array_equal(a, b, err_msg="forward repeat")
    dp2 = DevProblem(p, 256)
    c = dp2.forward().cpu().numpy()
    np.testing.assert_array_equal(a, c, err_msg="forward with a fresh plan")
    d1 = [x.cpu().numpy() for x in dp.backward()]
    d2 = [x.cpu().numpy() for x in dp.backward()]
    for k in range(3):
        assert_close(d2[k], d1[k].astype(np.float64), f"backward repeat dG{k + 1}")


# ---------------------------------------------------------------------------
# backward + SGD

def _check_backward(p, label, chunk=256, mask=None, slices=None):
    say(label, f"backward L={p.L} chunk={chunk}")
    dp = DevProblem(p, chunk)
    d = [x.cpu().numpy() for x in dp.backward()]
    ref = oracle.backward_problem(p, mask=mask)
    names = ("dG1", "dG2", "dG3")
    for k in range(3):
        if slices is None:
            assert_close(d[k], ref[k], f"{label} {names[k]}")
        else:
            sel = slices[k]
            assert_close(d[k][sel], ref[k][sel], f"{label} {names[k]} (sampled)")
    # SGD on the GPU from the GPU gradients, against the oracle's update
    from tensor_train_compressed_amd import tt_emb_sgd
    dg = dp.backward()
    g = [dp.g1.clone(), dp.g2.clone(), dp.g3.clone()]
    tt_emb_sgd(dp.plan, g[0], g[1], g[2], dg[0], dg[1], dg[2], p.lr)
    cores = (p.g1, p.g2, p.g3)
    for k in range(3):
        want = oracle.sgd(cores[k], ref[k], p.lr)
        got = g[k].cpu().numpy()
        sel = slice(None) if slices is None else slices[k]
        assert_close(got[sel], want[sel], f"{label} SGD core {k + 1}")


def test_backward_small_all():
    p = wl.make("train11m", batch=256)
    for chunk in (1, 7, 256):
        _check_backward(p, f"train11m B=256", chunk=chunk)


def test_backward_unaligned_dg2():
    """dG2 written through a pointer 4 bytes past a 16-byte boundary (the
    library takes any 4-byte-aligned output): the result still matches the
    oracle."""
    import tensor_train_compressed_amd as tte
    p = wl.make("train11m", batch=256)
    dp = DevProblem(p, 256)
    dp.make_plan()
    d1 = torch.empty_like(dp.g1)
    d3 = torch.empty_like(dp.g3)
    buf = torch.empty(dp.g2.numel() + 4, dtype=torch.float32, device="cuda:0")
    d2 = buf[1:1 + dp.g2.numel()]
    assert d2.data_ptr() % 16 == 4
    tte.tt_emb_backward(dp.plan, dp.g1, dp.g2, dp.g3, dp.gout, d1, d2, d3)
    ref = oracle.backward_problem(p)
    for k, x in enumerate((d1, d2, d3)):
        assert_close(x.cpu().numpy(), ref[k], f"unaligned dG2: dG{k + 1}")


def _oracle_backward_sgd(p):
    ref = oracle.backward_problem(p)
    return ref, [oracle.sgd(c, r, p.lr) for c, r in zip((p.g1, p.g2, p.g3), ref)]


def test_forward_train_token():
    """tt_emb_forward_train gives the forward's output bit for bit and a
    token; tt_emb_backward_kept with it matches the oracle. The token names
    one use of the kept products: a second backward_kept, one after an SGD
    step, after a plain backward (which overwrites them), after a newer
    forward_train, or with other core pointers gets TT_ERR_STALE and
    launches nothing."""
    import tensor_train_compressed_amd as tte
    p = wl.make("train11m", batch=1024)
    dp = DevProblem(p, 256)
    want_out = dp.forward().cpu().numpy()
    out = torch.empty(want_out.shape, dtype=torch.float32, device="cuda:0")
    d = [torch.empty_like(x) for x in (dp.g1, dp.g2, dp.g3)]
    g = (dp.g1, dp.g2, dp.g3)

    def stale(fn):
        with pytest.raises(tte.TTEmbError) as ei:
            fn()
        assert ei.value.status == tte.TT_ERR_STALE

    tok = tte.tt_emb_forward_train(dp.plan, *g, out)
    assert tok != 0
    np.testing.assert_array_equal(out.cpu().numpy(), want_out, err_msg="forward_train output")
    tte.tt_emb_backward_kept(dp.plan, tok, *g, dp.gout, *d)
    ref, ref_sgd = _oracle_backward_sgd(p)
    for k in range(3):
        assert_close(d[k].cpu().numpy(), ref[k], f"backward_kept dG{k + 1}")
    stale(lambda: tte.tt_emb_backward_kept(dp.plan, tok, *g, dp.gout, *d))       # consumed
    # a newer forward_train invalidates the older token
    t1 = tte.tt_emb_forward_train(dp.plan, *g, out)
    t2 = tte.tt_emb_forward_train(dp.plan, *g, out)
    assert t1 != t2
    stale(lambda: tte.tt_emb_backward_kept(dp.plan, t1, *g, dp.gout, *d))
    # other core pointers (same values)
    g1c = dp.g1.clone()
    stale(lambda: tte.tt_emb_backward_kept(dp.plan, t2, g1c, dp.g2, dp.g3, dp.gout, *d))
    # forward_train(A), backward on other cores B (plain: forms B's products
    # over the kept ones), then backward_kept(A's token): stale; a plain
    # backward on A is still right
    t3 = tte.tt_emb_forward_train(dp.plan, *g, out)
    gb = [x * 1.5 for x in g]
    db = [torch.empty_like(x) for x in g]
    tte.tt_emb_backward(dp.plan, *gb, dp.gout, *db)
    stale(lambda: tte.tt_emb_backward_kept(dp.plan, t3, *g, dp.gout, *d))
    tte.tt_emb_backward(dp.plan, *g, dp.gout, *d)
    for k in range(3):
        assert_close(d[k].cpu().numpy(), ref[k], f"plain backward after another core set dG{k + 1}")
    # an SGD step on the plan ends the token; then a second core set (the
    # oracle's cores after a step of lr 1e-4: fresh inputs for both sides; at
    # lr 0.01 the 1,024 bags' gradients, up to about 10^3, would blow the
    # cores up until fp32 rows lose the tolerance to cancellation) matches
    # the oracle again
    t4 = tte.tt_emb_forward_train(dp.plan, *g, out)
    tte.tt_emb_sgd(dp.plan, *[x.clone() for x in g], *d, p.lr)
    stale(lambda: tte.tt_emb_backward_kept(dp.plan, t4, *g, dp.gout, *d))
    new = [oracle.sgd(c, r, 1e-4).astype(np.float32) for c, r in zip((p.g1, p.g2, p.g3), ref)]
    p2 = wl.Problem(p.name, p.tables, p.batch, *new, p.goff, p.indices, p.offsets, p.grad_out, p.lr)
    for x, y in zip(g, (p2.g1, p2.g2, p2.g3)):
        x.copy_(torch.from_numpy(y))
    t5 = tte.tt_emb_forward_train(dp.plan, *g, out)
    assert_close(out.cpu().numpy(), oracle.forward_problem(p2), "forward_train on updated cores")
    tte.tt_emb_backward_kept(dp.plan, t5, *g, dp.gout, *d)
    ref2 = oracle.backward_problem(p2)
    for k in range(3):
        assert_close(d[k].cpu().numpy(), ref2[k], f"backward_kept on updated cores dG{k + 1}")


def test_training_step_full_size():
    """The step the benchmark times, at full size (the 11M-row table, 32,768
    bags, 656,601 lookups, chunk 256, one workspace for both steps): plan,
    tt_emb_forward_train, tt_emb_backward_kept, tt_emb_sgd. Every output row,
    every gradient element and every updated core element against the
    oracle; the step runs twice on the same workspace, each time from the
    workload's cores."""
    import tensor_train_compressed_amd as tte
    p = wl.make("train11m")
    dp = DevProblem(p, 256)
    ws = torch.empty(tte.tt_emb_workspace_bytes(dp.tables_c, p.L, p.batch, 256), dtype=torch.uint8,
                     device="cuda:0")
    say("full training step: oracle forward + backward (about a minute)")
    ref_out = oracle.forward_problem(p)
    ref, ref_sgd = _oracle_backward_sgd(p)
    # step 0: backward into gradient buffers, then tt_emb_sgd; step 1: the
    # fused tt_emb_backward_sgd (the benchmark's step), whose updated cores
    # must equal step 0's bit for bit
    first = None
    for step in range(2):
        g = [torch.from_numpy(x).to("cuda:0") for x in (p.g1, p.g2, p.g3)]
        d = [torch.empty_like(x) for x in g]
        out = torch.empty((p.batch, p.dim), dtype=torch.float32, device="cuda:0")
        pl = tte.tt_emb_plan(dp.tables_c, dp.idx, dp.off, p.batch, 256, workspace=ws)
        tok = tte.tt_emb_forward_train(pl, *g, out)
        assert tok != 0
        if step == 0:
            tte.tt_emb_backward_kept(pl, tok, *g, dp.gout, *d)
            tte.tt_emb_sgd(pl, *g, *d, p.lr)
        else:
            tte.tt_emb_backward_sgd(pl, tok, *g, dp.gout, p.lr)
        assert tte.tt_emb_get_error(pl) == 0
        say(f"step {step}: compare")
        assert_close(out.cpu().numpy(), ref_out, f"step {step} forward")
        for k in range(3):
            if step == 0:
                assert_close(d[k].cpu().numpy(), ref[k], f"step {step} dG{k + 1}")
            assert_close(g[k].cpu().numpy(), ref_sgd[k], f"step {step} SGD core {k + 1}")
        cores = [x.cpu().numpy() for x in g]
        if first is None:
            first = cores
        else:
            for k in range(3):
                np.testing.assert_array_equal(cores[k], first[k], err_msg=f"fused step core {k + 1}")


def test_query_paths():
    import tensor_train_compressed_amd as tte
    dp = DevProblem(wl.make("train11m", batch=64), 256)
    dp.make_plan()
    q = tte.tt_emb_query_paths(dp.plan, dp.g1, dp.g2)
    assert q["forward_path"] == tte.TT_PATH_MATRIX_CORE and q["backward_path"] == tte.TT_PATH_MATRIX_CORE
    assert q["keeps_prefix"] == 1 and q["dg3_by_rows"] == 1
    assert q["workspace_bytes"] == dp.plan.workspace.numel()
    # G1 at an address that is not 16-byte aligned: the generic kernels,
    # still matching the oracle
    buf = torch.empty(dp.g1.numel() + 1, dtype=torch.float32, device="cuda:0")
    g1u = buf[1:]
    g1u.copy_(dp.g1)
    q = tte.tt_emb_query_paths(dp.plan, g1u, dp.g2)
    assert q["forward_path"] == tte.TT_PATH_GENERIC and q["backward_path"] == tte.TT_PATH_GENERIC
    assert q["keeps_prefix"] == 0
    out = torch.empty((dp.TB, dp.D), dtype=torch.float32, device="cuda:0")
    assert tte.tt_emb_forward_train(dp.plan, g1u, dp.g2, dp.g3, out) == 0   # nothing kept
    assert_close(out.cpu().numpy(), oracle.forward_problem(dp.p), "generic forward (unaligned G1)")
    # a shape without matrix-core kernels
    tabs = [wl.Table(5000, (17, 18, 17), (4, 2, 1), 5)]
    dq = DevProblem(wl.make_custom(tabs, np.full(10, 3), seed=3), 16)
    dq.make_plan()
    q = tte.tt_emb_query_paths(dq.plan, dq.g1, dq.g2)
    assert q["forward_path"] == tte.TT_PATH_GENERIC and q["backward_path"] == tte.TT_PATH_GENERIC


def test_binding_checks_sizes():
    import tensor_train_compressed_amd as tte
    dp = DevProblem(wl.make("train11m", batch=64), 256)
    dp.make_plan()
    out = torch.empty((dp.TB, dp.D), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ValueError):
        tte.tt_emb_forward(dp.plan, dp.g1, dp.g2, dp.g3, out[:-1])
    with pytest.raises(ValueError):
        tte.tt_emb_forward(dp.plan, dp.g1[:-4], dp.g2, dp.g3, out)
    with pytest.raises(ValueError):
        tte.tt_emb_plan(dp.tables_c, dp.idx, dp.off[:-1], dp.p.batch, 256)
    d = [torch.empty_like(x) for x in (dp.g1, dp.g2, dp.g3)]
    with pytest.raises(ValueError):
        tte.tt_emb_backward(dp.plan, dp.g1, dp.g2, dp.g3, dp.gout, d[0], d[1][:-1], d[2])


def test_backward_multitable_small():
    p = wl.make("multi26", batch=32, tables=6)
    p.grad_out = np.random.default_rng(1).standard_normal((p.T * p.batch, p.dim)).astype(np.float32)
    p.lr = 0.01
    _check_backward(p, "multi26 6 tables B=32")


def test_backward_ragged():
    tabs = [wl.Table(97, (5, 4, 5), (2, 2, 2), 3), wl.Table(1, (1, 1, 1), (1, 8, 1), 2),
            wl.Table(5000, (17, 18, 17), (4, 2, 1), 5)]
    p = wl.make_custom(tabs, np.random.default_rng(0).integers(0, 9, 3 * 100), seed=4,
                       with_grad=True)
    for chunk in (1, 64):
        _check_backward(p, f"ragged chunk={chunk}", chunk=chunk)


@pytest.mark.parametrize("m3,pad3", [(1024, 0), (1025, 0), (1024, 4)])
def test_backward_g3_buckets(m3, pad3):
    # dG3 from the run rows bucketed by G3 row; with the table's G3 placed 4
    # floats into its buffer (rows not aligned to R*n3) it takes the device
    # atomics instead. L = 4097 lookups: one full sort tile and a ragged one;
    # Zipf indices so rows repeat inside groups.
    t = wl.Table(4 * 5 * m3, (4, 5, m3), (4, 8, 4), 32)
    lens = np.full(97, 42, np.int64)
    lens[-1] += 4097 - int(lens.sum())
    p = wl.make_custom([t], lens, seed=6, zipf_alpha=1.05, with_grad=True)
    assert p.L == 4097
    if pad3:
        p.g3 = np.concatenate([np.zeros(pad3, np.float32), p.g3])
        p.goff = p.goff.copy()
        p.goff[0, 2] = pad3
    _check_backward(p, f"m3={m3} G3 at {pad3} L=4097", chunk=64)


def test_backward_shared_g3_and_empty():
    # two tables reading one G3 (same offset): both tables' runs land in the
    # same dG3 buckets and the slices get both sums
    t1 = wl.Table(4 * 5 * 300, (4, 5, 300), (4, 8, 4), 32)
    t2 = wl.Table(3 * 6 * 300, (3, 6, 300), (4, 8, 4), 32)
    p = wl.make_custom([t1, t2], np.full(2 * 60, 7), seed=7, zipf_alpha=1.1, with_grad=True)
    p.g3 = p.g3[:300 * 32 * 4].copy()
    p.goff = p.goff.copy()
    p.goff[1, 2] = 0
    _check_backward(p, "shared G3", chunk=32)
    # no lookups at all: every gradient is zero
    q = wl.make_custom([t1], np.zeros(16, np.int64), seed=8, with_grad=True)
    assert q.L == 0
    _check_backward(q, "no lookups", chunk=32)


def test_backward_shared_g1_g2():
    # two tables reading one G1 and one G2 (same offsets), shapes of the
    # matrix-core path: each shared core's gradient is the sum of both tables'
    t1 = wl.Table(4 * 6 * 300, (4, 6, 300), (4, 8, 4), 32)
    t2 = wl.Table(4 * 6 * 200, (4, 6, 200), (4, 8, 4), 32)
    p = wl.make_custom([t1, t2], np.full(2 * 60, 7), seed=9, zipf_alpha=1.1, with_grad=True)
    p.g1 = p.g1[:4 * 4 * 32].copy()
    p.g2 = p.g2[:6 * 32 * 8 * 32].copy()
    p.goff = p.goff.copy()
    p.goff[1, 0] = 0
    p.goff[1, 1] = 0
    _check_backward(p, "shared G1 and G2", chunk=32)


def test_backward_multitable_full_size_sampled():
    """The 26-table batch at full size (8.5 M lookups): dG3 through buckets of
    2,391 G3 rows, the planner's scans past 512 tiles. In each of the three
    largest tables one slice of each core (cold under the unpermuted Zipf
    head) is compared, against the oracle run on the lookups touching them
    (exact for those slices)."""
    p = wl.make("multi26")
    p.grad_out = np.random.default_rng(2).standard_normal((p.T * p.batch, p.dim)).astype(np.float32)
    p.lr = 0.01
    pl = oracle.plan_problem(p, 256)
    kb = np.cumsum([0] + [t.m[0] * t.m[1] for t in p.tables])
    key = pl["key"].astype(np.int64)
    i3 = pl["i3"].astype(np.int64)
    tab = np.searchsorted(kb, key, side="right") - 1
    m1 = np.array([t.m[0] for t in p.tables])
    i1 = (key - kb[tab]) % m1[tab]
    i2 = (key - kb[tab]) // m1[tab]
    mask = np.zeros(p.L, bool)
    s1, s2, s3 = [], [], []
    for t in np.argsort([-t.num_rows for t in p.tables])[:3]:
        tb = p.tables[t]
        R, (n1, n2, n3) = tb.rank, tb.n
        a1, a2, a3 = tb.m[0] - 1, tb.m[1] // 2, tb.m[2] // 3
        mask |= (tab == t) & ((i1 == a1) | (i2 == a2) | (i3 == a3))
        o1, o2, o3 = p.goff[t]
        s1.append(np.arange(o1 + a1 * n1 * R, o1 + (a1 + 1) * n1 * R))
        s2.append(np.arange(o2 + a2 * R * n2 * R, o2 + (a2 + 1) * R * n2 * R))
        s3.append(np.arange(o3 + a3 * R * n3, o3 + (a3 + 1) * R * n3))
    say("sampled multitable backward lookups", int(mask.sum()))
    _check_backward(p, "multi26 full (sampled)", chunk=256, mask=mask.astype(np.uint8),
                    slices=(np.concatenate(s1), np.concatenate(s2), np.concatenate(s3)))


def test_backward_piece_list_overflow():
    """More pieces of large groups than the piece list holds (8,192): 300
    groups of 1,024 distinct rows each (32 pieces per group, 9,600 in all),
    so the groups that do not fit run whole on one wave each; every
    gradient element against the oracle. Shape (4, 4, 4), R 32: each run's
    dG3 term (128 floats) is longer than its S row (64), so it goes to a
    buffer of its own."""
    t = wl.Table(20 * 15 * 1024, (20, 15, 1024), (4, 4, 4), 32)
    L = 20 * 15 * 1024
    p = wl.make_custom([t], np.full(L // 100, 100), seed=11, with_grad=True)
    assert p.L == L
    p.indices = np.random.default_rng(12).permutation(L).astype(np.int64)
    _check_backward(p, "piece list overflow (9,600 pieces)", chunk=256)


def test_backward_hot_slices_full_size():
    """train11m at full size, the hottest slices (i1 = 0, i2 = 0, i3 = 0):
    against the fp64 oracle's values stored by
    tests/golden/make_train11m_hot_slices.py (the oracle on these slices takes
    about a minute, too long to rerun here). Two runs: the fp64 accumulation
    order differs between them."""
    from tests.golden.make_train11m_hot_slices import OUT, fingerprint
    g = np.load(OUT)
    p = wl.make("train11m")
    assert str(g["fingerprint"]) == fingerprint(p), \
        "train11m inputs changed: rerun tests/golden/make_train11m_hot_slices.py"
    t = p.tables[0]
    R, (n1, n2, n3) = t.rank, t.n
    dp = DevProblem(p, 256)
    for run in range(2):
        d = [x.cpu().numpy() for x in dp.backward()]
        assert_close(d[0][:n1 * R], g["dg1_i1_0"], f"hot dG1[i1=0] run {run}")
        assert_close(d[1][:R * n2 * R], g["dg2_i2_0"], f"hot dG2[i2=0] run {run}")
        assert_close(d[2][:R * n3], g["dg3_i3_0"], f"hot dG3[i3=0] run {run}")


def test_kernel_timing():
    """tt_emb_set_timing brackets every launch with events: a forward records
    the G3 transpose, batch and pooling kernels once each, with positive times; a plan made
    while the process-wide default is on records its planning kernels."""
    import tensor_train_compressed_amd as tte
    dp = DevProblem(wl.make("train11m", batch=256), 256)
    tte.tt_emb_set_timing(None, True)
    try:
        pl = tte.tt_emb_plan(dp.tables_c, dp.idx, dp.off, dp.p.batch, 256)
    finally:
        tte.tt_emb_set_timing(None, False)
    names = [k for k, _ in tte.tt_emb_kernel_times(pl)]
    assert "k_split" in names and "k_batches" in names and "k_radix_scatter" in names
    out = torch.empty((dp.TB, dp.D), dtype=torch.float32, device="cuda:0")
    tte.tt_emb_forward(pl, dp.g1, dp.g2, dp.g3, out)
    t = tte.tt_emb_kernel_times(pl)
    assert [k for k, _ in t] == ["k_g3t", "k_fwd_batch", "k_pool"] and all(ms > 0 for _, ms in t)
    tte.tt_emb_set_timing(pl, False)
    tte.tt_emb_forward(pl, dp.g1, dp.g2, dp.g3, out)
    assert tte.tt_emb_kernel_times(pl) == []
    assert_close(out.cpu().numpy(), oracle.forward_problem(dp.p), "forward with timing toggled")


@pytest.mark.parametrize("case", ["single", "multi6", "shared_g3", "no_lookups", "recompute", "gap_g2"])
def test_backward_sgd_fused(case):
    """tt_emb_backward_sgd against tt_emb_backward + tt_emb_sgd on the same
    inputs: the updated cores bit for bit (untouched slices unchanged), and
    against the oracle's step; with a kept token and (recompute) without;
    gap_g2: the second table's G2 slices start 1,000 floats past the first's
    end (the gap belongs to no table and must keep its values)."""
    import tensor_train_compressed_amd as tte
    if case == "single":
        p = wl.make("train11m", batch=256)
    elif case == "recompute":
        p = wl.make("train11m", batch=300)
    elif case == "multi6":
        p = wl.make("multi26", batch=32, tables=6)
        p.grad_out = np.random.default_rng(1).standard_normal((p.T * p.batch, p.dim)).astype(np.float32)
        p.lr = 0.01
    elif case == "gap_g2":
        t1 = wl.Table(20 * 30 * 40, (20, 30, 40), (4, 8, 4), 32)
        t2 = wl.Table(25 * 12 * 40, (25, 12, 40), (4, 8, 4), 32)
        p = wl.make_custom([t1, t2], np.full(2 * 64, 9), seed=11, zipf_alpha=1.1, with_grad=True)
        gap, e1 = 1000, int(p.goff[1, 1])
        g2 = np.random.default_rng(5).standard_normal(p.g2.size + gap).astype(np.float32)
        g2[:e1] = p.g2[:e1]
        g2[e1 + gap:] = p.g2[e1:]
        p.g2 = g2
        p.goff = p.goff.copy()
        p.goff[1, 1] += gap
    else:
        t1 = wl.Table(4 * 5 * 300, (4, 5, 300), (4, 8, 4), 32)
        t2 = wl.Table(3 * 6 * 300, (3, 6, 300), (4, 8, 4), 32)
        lens = np.full(2 * 60, 7) if case == "shared_g3" else np.zeros(2 * 16, np.int64)
        p = wl.make_custom([t1, t2], lens, seed=7, zipf_alpha=1.1, with_grad=True)
        p.g3 = p.g3[:300 * 32 * 4].copy()
        p.goff = p.goff.copy()
        p.goff[1, 2] = 0
    dp = DevProblem(p, 32)
    dp.make_plan()
    if case == "gap_g2":   # the matrix-core backward, with its dG2 buffer over a gapped G2
        assert tte.tt_emb_query_paths(dp.plan, dp.g1, dp.g2)["backward_path"] == 1
    out = torch.empty((dp.TB, dp.D), dtype=torch.float32, device="cuda:0")
    g = [x.clone() for x in (dp.g1, dp.g2, dp.g3)]
    d = [torch.empty_like(x) for x in g]
    tok = tte.tt_emb_forward_train(dp.plan, *g, out)
    if tok:
        tte.tt_emb_backward_kept(dp.plan, tok, *g, dp.gout, *d)
    else:   # no lookups: nothing is kept
        assert p.L == 0
        tte.tt_emb_backward(dp.plan, *g, dp.gout, *d)
    tte.tt_emb_sgd(dp.plan, *g, *d, p.lr)
    want = [x.cpu().numpy() for x in g]
    f = [x.clone() for x in (dp.g1, dp.g2, dp.g3)]
    tok = tte.tt_emb_forward_train(dp.plan, *f, out) if case != "recompute" else 0
    tte.tt_emb_backward_sgd(dp.plan, tok, *f, dp.gout, p.lr)
    ref, ref_sgd = _oracle_backward_sgd(p)
    touched = [np.asarray(r) != 0 for r in ref]
    for k in range(3):
        got = f[k].cpu().numpy()
        np.testing.assert_array_equal(got, want[k], err_msg=f"{case}: fused core {k + 1}")
        assert_close(got, ref_sgd[k], f"{case}: fused core {k + 1} vs oracle")
        orig = (p.g1, p.g2, p.g3)[k]
        np.testing.assert_array_equal(got[~touched[k]], orig[~touched[k]], err_msg=f"{case}: untouched {k + 1}")
    # a stale token is refused before any launch, the cores untouched
    with pytest.raises(tte.TTEmbError) as ei:
        tte.tt_emb_backward_sgd(dp.plan, 12345, *f, dp.gout, p.lr)
    assert ei.value.status == tte.TT_ERR_STALE


def test_pipelined_steps_match_serial():
    """Training steps on four different batches, run one after another on one
    stream, and run as the benchmark runs them: each batch's plan built on a
    second stream into the other of two workspaces while the previous batch
    computes. The cores after the last step and its forward output agree bit
    for bit (plans on separate workspaces share no device state)."""
    import tensor_train_compressed_amd as tte
    base = wl.make("train11m", batch=2048)
    batches = [wl.make("train11m", seed=s, batch=2048) for s in (1, 2, 3, 4)]
    tabs = tte.make_tables(base.tables, base.goff)
    dev = "cuda:0"
    ins = [(torch.from_numpy(b.indices).to(dev), torch.from_numpy(b.offsets).to(dev),
            torch.from_numpy(b.grad_out).to(dev)) for b in batches]
    nws = tte.tt_emb_workspace_bytes(tabs, max(b.L for b in batches), 2048, 256)
    wss = [torch.empty(nws, dtype=torch.uint8, device=dev) for _ in range(2)]
    out = torch.empty((2048, base.dim), dtype=torch.float32, device=dev)

    def cores():
        return [torch.from_numpy(x).to(dev) for x in (base.g1, base.g2, base.g3)]

    g = cores()
    for idx, off, gout in ins:
        pl = tte.tt_emb_plan(tabs, idx, off, 2048, 256, workspace=wss[0])
        tok = tte.tt_emb_forward_train(pl, *g, out)
        tte.tt_emb_backward_sgd(pl, tok, *g, gout, base.lr)
    torch.cuda.synchronize()
    want = [x.cpu().numpy() for x in g] + [out.cpu().numpy()]

    out.fill_(0)
    g = cores()
    sc, sp = torch.cuda.current_stream(), torch.cuda.Stream()
    planned = [torch.cuda.Event(), torch.cuda.Event()]
    used = [torch.cuda.Event(), torch.cuda.Event()]
    plans = [None, None]
    sp.wait_stream(sc)
    plans[0] = tte.tt_emb_plan(tabs, ins[0][0], ins[0][1], 2048, 256, workspace=wss[0], stream=sp)
    planned[0].record(sp)
    for i in range(len(ins)):
        c, n = i % 2, (i + 1) % 2
        sc.wait_event(planned[c])
        tok = tte.tt_emb_forward_train(plans[c], *g, out, stream=sc)
        tte.tt_emb_backward_sgd(plans[c], tok, *g, ins[i][2], base.lr, stream=sc)
        used[c].record(sc)
        if i + 1 < len(ins):
            if i >= 1:
                sp.wait_event(used[n])
            plans[n] = tte.tt_emb_plan(tabs, ins[i + 1][0], ins[i + 1][1], 2048, 256, workspace=wss[n], stream=sp)
            planned[n].record(sp)
    torch.cuda.synchronize()
    assert tte.tt_emb_get_error(plans[(len(ins) - 1) % 2]) == 0
    got = [x.cpu().numpy() for x in g] + [out.cpu().numpy()]
    for k, name in enumerate(("G1", "G2", "G3", "last forward")):
        np.testing.assert_array_equal(got[k], want[k], err_msg=name)


# (n1, n2, n3, R, backward on the matrix cores too): every shape the
# matrix-core kernels are built for, beyond the benchmark's (4, 8, 4, 32)
MFMA_SHAPES = [(4, 4, 4, 32, True), (4, 4, 4, 16, True), (2, 8, 4, 32, True), (8, 4, 4, 32, True),
               (4, 4, 4, 64, True), (4, 4, 8, 32, False), (4, 4, 2, 32, False), (4, 4, 1, 32, False)]


@pytest.mark.parametrize("n1,n2,n3,R,bw", MFMA_SHAPES)
def test_matrix_core_shapes(n1, n2, n3, R, bw):
    """Each built shape runs on the matrix-core kernels (query) and matches
    the oracle on every output element; shapes with a matrix-core backward
    also match on every gradient element, through the kept prefixes, the
    recomputed ones and the fused SGD step. 300 Zipf-skewed bags over a
    7,200-row table: groups of many runs (split into pieces in the
    backward), batches of up to 8 groups, ragged tiles."""
    import tensor_train_compressed_amd as tte
    t = wl.Table(20 * 12 * 30, (20, 12, 30), (n1, n2, n3), R)
    lens = np.random.default_rng(3).poisson(12, 300)
    p = wl.make_custom([t], lens, seed=12, zipf_alpha=1.05, with_grad=True)
    label = f"shape ({n1},{n2},{n3}) R={R} L={p.L}"
    dp = DevProblem(p, 64)
    dp.make_plan()
    q = tte.tt_emb_query_paths(dp.plan, dp.g1, dp.g2)
    assert q["forward_path"] == tte.TT_PATH_MATRIX_CORE, label
    assert q["backward_path"] == (tte.TT_PATH_MATRIX_CORE if bw else tte.TT_PATH_GENERIC), label
    out = torch.empty((dp.TB, dp.D), dtype=torch.float32, device="cuda:0")
    tok = tte.tt_emb_forward_train(dp.plan, dp.g1, dp.g2, dp.g3, out)
    assert (tok != 0) == bw, label
    say(label, "forward")
    assert_close(out.cpu().numpy(), oracle.forward_problem(p), f"{label} forward")
    ref = oracle.backward_problem(p)
    d = [torch.empty_like(x) for x in (dp.g1, dp.g2, dp.g3)]
    if bw:
        say(label, "backward (kept prefixes)")
        tte.tt_emb_backward_kept(dp.plan, tok, dp.g1, dp.g2, dp.g3, dp.gout, *d)
        for k in range(3):
            assert_close(d[k].cpu().numpy(), ref[k], f"{label} kept dG{k + 1}")
    say(label, "backward")
    tte.tt_emb_backward(dp.plan, dp.g1, dp.g2, dp.g3, dp.gout, *d)
    for k in range(3):
        assert_close(d[k].cpu().numpy(), ref[k], f"{label} dG{k + 1}")
    if bw:
        say(label, "fused backward + SGD")
        g = [x.clone() for x in (dp.g1, dp.g2, dp.g3)]
        tok = tte.tt_emb_forward_train(dp.plan, *g, out)
        tte.tt_emb_backward_sgd(dp.plan, tok, *g, dp.gout, p.lr)
        for k, (c, r) in enumerate(zip((p.g1, p.g2, p.g3), ref)):
            assert_close(g[k].cpu().numpy(), oracle.sgd(c, r, p.lr), f"{label} fused SGD core {k + 1}")


def _top_pairs(p, k):
    """The k most frequent (table, row) pairs of the batch."""
    bag = np.repeat(np.arange(p.T * p.batch), np.diff(p.offsets))
    key = (bag // p.batch) * (1 << 40) + p.indices
    u, c = np.unique(key, return_counts=True)
    top = u[np.argsort(-c, kind="stable")[:k]]
    return (top >> 40).astype(np.int32), (top & ((1 << 40) - 1)).astype(np.int64)


@pytest.mark.parametrize("case", ["single", "multi6", "empty", "all_hot", "no_lookups"])
def test_hot_row_cache(case):
    """Hot rows kept uncompressed (the TT-Rec cache): forward, backward (kept
    and recomputed prefixes) and the fused step against the oracle's cached
    model on every element; a cache holding the rows' own TT values gives the
    plain forward; the plain calls refuse a cached plan and the reverse."""
    import tensor_train_compressed_amd as tte
    if case == "multi6":
        p = wl.make("multi26", batch=32, tables=6)
        p.grad_out = np.random.default_rng(1).standard_normal((p.T * p.batch, p.dim)).astype(np.float32)
        p.lr = 0.01
    elif case == "no_lookups":
        t = wl.Table(4 * 5 * 300, (4, 5, 300), (4, 8, 4), 32)
        p = wl.make_custom([t], np.zeros(16, np.int64), seed=7, with_grad=True)
    else:
        p = wl.make("train11m", batch=512)
    if case == "empty":
        ht, hr = np.zeros(0, np.int32), np.zeros(0, np.int64)
    elif case == "all_hot":   # every row the batch looks up is hot: the cores get no gradient
        ht, hr = _top_pairs(p, 1 << 30)
    elif case == "no_lookups":
        ht, hr = np.array([0, 0], np.int32), np.array([3, 4], np.int64)
    else:
        ht, hr = _top_pairs(p, 96)
        # a duplicate (served by its first slot) and a pair naming no row
        ht = np.concatenate([ht, ht[:1], [0]]).astype(np.int32)
        hr = np.concatenate([hr, hr[:1], [p.tables[0].num_rows + 5]]).astype(np.int64)
    n = hr.size
    say(case, f"L={p.L} hot entries={n}")
    dp = DevProblem(p, 64)
    cache = tte.HotCache(torch.from_numpy(ht).to("cuda:0"), torch.from_numpy(hr).to("cuda:0"))
    plan = tte.tt_emb_plan(dp.tables_c, dp.idx, dp.off, p.batch, 64, cache=cache)
    W = np.random.default_rng(2).standard_normal((n, p.dim)).astype(np.float32)
    Wd = torch.from_numpy(W).to("cuda:0")
    out = torch.empty((dp.TB, dp.D), dtype=torch.float32, device="cuda:0")
    tok = tte.tt_emb_forward_cached(plan, dp.g1, dp.g2, dp.g3, Wd, out, keep=True)
    assert (tok != 0) == (p.L > 0)
    assert_close(out.cpu().numpy(), oracle.forward_cached(p, ht, hr, W), f"{case}: cached forward")
    ref = oracle.backward_cached(p, ht, hr, n)
    d = [torch.empty_like(x) for x in (dp.g1, dp.g2, dp.g3)]
    dW = torch.full_like(Wd, 7.0)
    for t in (tok, 0):
        tte.tt_emb_backward_cached(plan, t, dp.g1, dp.g2, dp.g3, dp.gout, *d, dW)
        for k in range(3):
            assert_close(d[k].cpu().numpy(), ref[k], f"{case}: cached dG{k + 1} (token {t})")
        assert_close(dW.cpu().numpy(), ref[3], f"{case}: dW (token {t})")
    # the fused step: cores and hot rows updated in place
    g = [x.clone() for x in (dp.g1, dp.g2, dp.g3)]
    Wf = Wd.clone()
    tok = tte.tt_emb_forward_cached(plan, *g, Wf, out, keep=True)
    tte.tt_emb_backward_sgd_cached(plan, tok, *g, Wf, dp.gout, p.lr)
    for k, c in enumerate((p.g1, p.g2, p.g3)):
        assert_close(g[k].cpu().numpy(), oracle.sgd(c, ref[k], p.lr), f"{case}: fused core {k + 1}")
    assert_close(Wf.cpu().numpy(), oracle.sgd(W, ref[3], p.lr), f"{case}: fused hot rows")
    # a cache holding the rows' own TT values: the plain model's output
    if case in ("all_hot", "no_lookups"):
        Wt = torch.from_numpy(oracle.materialise_rows(p, ht, hr).astype(np.float32)).to("cuda:0")
    elif n:
        Wt = torch.from_numpy(oracle.materialise_rows(p, ht[:-1], hr[:-1]).astype(np.float32))
        Wt = torch.cat([Wt, torch.zeros(1, p.dim)]).to("cuda:0")
    else:
        Wt = Wd
    tte.tt_emb_forward_cached(plan, dp.g1, dp.g2, dp.g3, Wt, out)
    assert_close(out.cpu().numpy(), oracle.forward_problem(p), f"{case}: TT-valued cache")
    # the plain calls refuse the cached plan, the cached ones a plain plan
    with pytest.raises(tte.TTEmbError) as ei:
        tte.tt_emb_forward(plan, dp.g1, dp.g2, dp.g3, out)
    assert ei.value.status == tte.TT_ERR_CACHE
    dp.make_plan()
    with pytest.raises(tte.TTEmbError) as ei:
        tte.tt_emb_backward_cached(dp.plan, 0, dp.g1, dp.g2, dp.g3, dp.gout, *d, dW)
    assert ei.value.status == tte.TT_ERR_CACHE


def test_generic_path_realistic_size():
    """A shape without matrix-core kernels (rank 12) at a realistic size
    (1M rows, 4,096 Zipf-skewed bags of Poisson(20) lookups): the query
    reports the generic kernels, and forward and backward match the oracle
    on every element."""
    import tensor_train_compressed_amd as tte
    t = wl.Table(100 ** 3, (100, 100, 100), (4, 4, 4), 12)
    lens = np.minimum(np.random.default_rng(5).poisson(20, 4096), 100)
    p = wl.make_custom([t], lens, seed=13, zipf_alpha=1.05, with_grad=True)
    dp = DevProblem(p, 256)
    dp.make_plan()
    q = tte.tt_emb_query_paths(dp.plan, dp.g1, dp.g2)
    assert q["forward_path"] == tte.TT_PATH_GENERIC and q["backward_path"] == tte.TT_PATH_GENERIC
    say("generic path", f"L={p.L}")
    assert_close(dp.forward().cpu().numpy(), oracle.forward_problem(p), "generic forward")
    ref = oracle.backward_problem(p)
    for k, x in enumerate(dp.backward()):
        assert_close(x.cpu().numpy(), ref[k], f"generic dG{k + 1}")
