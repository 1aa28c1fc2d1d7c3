"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import tensor_train_compressed_amd as tte

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(tte.library_path()):
        pytest.fail("libtt_emb.so is not built (run __graft_entry__.build())")
    return tte.load_library()


def test_header_declarations_are_exported():
    hdr = open(os.path.join(ROOT, "include", "tt_emb.h")).read()
    declared = set(re.findall(r"\b(tt_emb_[a-z_]+)\s*\(", hdr))
    assert declared == set(tte.EXPORTS)
    lib = _lib()
    for name in declared:
        assert hasattr(lib, name), name


class _T:
    def __init__(self, N, m, n, R):
        self.num_rows, self.m, self.n, self.rank = N, m, n, R


def _tabs(*specs):
    ts = [_T(*s) for s in specs]
    return tte.make_tables(ts, [(0, 0, 0)] * len(ts))


def test_workspace_bytes_host_validation():
    _lib()
    good = _tabs((11_000_000, (200, 220, 250), (4, 8, 4), 32))
    assert tte.tt_emb_workspace_bytes(good, 655_000, 32768, 256) > 655_000 * 4 * 7
    assert tte.tt_emb_workspace_bytes(good, 0, 32768, 256) > 0          # empty batch is fine
    assert tte.tt_emb_workspace_bytes(good, 10, 32768, 0) == 0          # chunk < 1
    assert tte.tt_emb_workspace_bytes(good, -1, 32768, 256) == 0
    assert tte.tt_emb_workspace_bytes(_tabs((1001, (10, 10, 10), (2, 2, 4), 4)), 1, 1, 1) == 0  # N > rows
    assert tte.tt_emb_workspace_bytes(_tabs((10, (10, 1, 1), (2, 2, 4), 65)), 1, 1, 1) == 0     # R > 64
    mixed = _tabs((10, (10, 1, 1), (2, 2, 4), 4), (10, (10, 1, 1), (4, 4, 4), 4))              # D differs
    assert tte.tt_emb_workspace_bytes(mixed, 1, 1, 1) == 0
    same_d = _tabs((10, (10, 1, 1), (2, 2, 4), 4), (10, (10, 1, 1), (4, 1, 4), 8))
    assert tte.tt_emb_workspace_bytes(same_d, 1, 1, 1) > 0
    assert tte.tt_emb_workspace_bytes(good, 5, 0, 16) == 0              # lookups but no bags


def test_plan_rejects_bad_args_before_launch():
    lib = _lib()
    good = _tabs((1000, (10, 10, 10), (2, 2, 4), 4))
    h = ctypes.c_void_p()
    P = ctypes.c_void_p
    # null plan_out, null offsets, misaligned/too-small workspace: all host-side
    assert lib.tt_emb_plan(good, 1, P(16), P(16), 4, 4, 8, P(256), 1 << 20, None, None) == -1
    assert lib.tt_emb_plan(good, 1, P(16), None, 4, 4, 8, P(256), 1 << 20, None, ctypes.byref(h)) == -1
    assert lib.tt_emb_plan(good, 1, P(16), P(16), 4, 4, 8, P(260), 1 << 20, None, ctypes.byref(h)) == -1
    assert lib.tt_emb_plan(good, 1, P(16), P(16), 4, 4, 8, P(256), 16, None, ctypes.byref(h)) == -3
    assert lib.tt_emb_plan(good, 0, P(16), P(16), 4, 4, 8, P(256), 1 << 20, None, ctypes.byref(h)) == -1
    assert h.value is None
    # null handles
    assert lib.tt_emb_forward(None, P(1), P(1), P(1), P(1), None) == -1
    assert lib.tt_emb_backward(None, P(1), P(1), P(1), P(1), P(1), P(1), P(1), None) == -1
    assert lib.tt_emb_sgd(None, P(1), P(1), P(1), P(1), P(1), P(1), ctypes.c_float(0.1), None) == -1
    tok = ctypes.c_uint64(7)
    assert lib.tt_emb_forward_train(None, P(1), P(1), P(1), P(1), ctypes.byref(tok), None) == -1
    assert tok.value == 0                      # no products kept
    assert lib.tt_emb_backward_kept(None, 1, P(1), P(1), P(1), P(1), P(1), P(1), P(1), None) == -1
    assert lib.tt_emb_query_paths(None, P(16), P(16), None) == -1
    assert lib.tt_emb_plan_destroy(None) == 0
    assert b"workspace" in lib.tt_emb_status_string(-3)
    assert b"stale" in lib.tt_emb_status_string(-6)


def test_workspace_size_skew11m():
    """The 11M-row table's batch (656,601 lookups, 32,768 bags) plans in
    under 700 MB of workspace."""
    _lib()
    good = _tabs((11_000_000, (200, 220, 250), (4, 8, 4), 32))
    assert tte.tt_emb_workspace_bytes(good, 656_601, 32768, 256) < 700e6


def test_more_entry_points_reject_bad_args_on_host():
    lib = _lib()
    P = ctypes.c_void_p
    assert lib.tt_emb_backward_sgd(None, 1, P(1), P(1), P(1), P(1), ctypes.c_float(0.1), None) == -1
    n = ctypes.c_int32(-1)
    assert lib.tt_emb_kernel_times(None, None, 0, ctypes.byref(n), None) == -1
    assert lib.tt_emb_set_timing(None, 1) == 0 and lib.tt_emb_set_timing(None, 0) == 0
    assert lib.tt_emb_scratch_capacity() == 64 << 20
    big = _tabs((11_000_000, (200, 220, 250), (4, 8, 4), 32))
    # a batch beyond the static buffer is refused before any device call
    assert lib.tt_emb_forward_scratch(big, 1, P(16), P(16), 2_000_000, 32768, 256,
                                      P(16), P(16), P(16), P(16), None) == -7
    # a batch that fits, with a null core: refused before the buffer is touched
    assert lib.tt_emb_forward_scratch(big, 1, P(16), P(16), 1000, 64, 256,
                                      None, P(16), P(16), P(16), None) == -1
    assert b"scratch" in lib.tt_emb_status_string(-7)
