"""The allocation-free forward (tt_emb_forward_scratch), through the C ABI:
its output against tt_emb_plan + tt_emb_forward on the same inputs (the same
kernels: bit for bit) and against the CPU oracle (within 1e-4 * (1 + |ref|)),
on two calls in a row, the second with a smaller batch; a batch too large for
the static buffer is refused before any device work."""
import numpy as np
import pytest

import oracle
import tensor_train_compressed_amd as tte
import workloads as wl

torch = pytest.importorskip("torch")


def _tables(p):
    return tte.make_tables(p.tables, p.goff)


@pytest.mark.gpu
def test_forward_scratch_matches_workspace_path():
    from tests.gpu_helpers import DevProblem, assert_close, say
    # two calls in a row on one device: a larger batch, then a smaller one
    # (the buffer keeps the first call's contents)
    for name, batch in (("skew11m", 3000), ("skew11m", 700)):
        p = wl.make(name, batch=batch)
        say("forward_scratch", name, batch, f"L={p.L}")
        dp = DevProblem(p, 256)
        want = dp.forward()
        got = torch.full_like(want, float("nan"))
        tte.tt_emb_forward_scratch(dp.tables_c, dp.idx, dp.off, p.batch, 256, dp.g1, dp.g2, dp.g3, got)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), want.cpu().numpy(), err_msg=f"{name} B={batch}")
        assert_close(got.cpu().numpy(), oracle.forward_problem(p), f"{name} B={batch} vs oracle")
    # a multi-table batch (generic-free matrix-core path, several tables)
    p = wl.make("multi26", batch=64, tables=5)
    dp = DevProblem(p, 256)
    want = dp.forward()
    got = torch.full_like(want, float("nan"))
    tte.tt_emb_forward_scratch(dp.tables_c, dp.idx, dp.off, p.batch, 256, dp.g1, dp.g2, dp.g3, got)
    np.testing.assert_array_equal(got.cpu().numpy(), want.cpu().numpy(), err_msg="multi-table")


def test_forward_scratch_refuses_large_batch():
    """Host-side: a batch needing more than the buffer gets TT_ERR_SCRATCH
    before any device call (works without a GPU)."""
    lib = tte.load_library()
    t = wl.Table(11_000_000, (200, 220, 250), (4, 8, 4), 32)
    tabs = tte.make_tables([t], [(0, 0, 0)])
    import ctypes
    P = ctypes.c_void_p
    cap = tte.tt_emb_scratch_capacity()
    assert cap == 64 << 20
    # 656,601 lookups of dim 128 need far more than 64 MiB
    st = lib.tt_emb_forward_scratch(tabs, 1, P(256), P(256), 656_601, 32768, 256, P(256), P(256), P(256),
                                    P(256), None)
    assert st == tte.TT_ERR_SCRATCH
    assert b"scratch" in lib.tt_emb_status_string(tte.TT_ERR_SCRATCH)
