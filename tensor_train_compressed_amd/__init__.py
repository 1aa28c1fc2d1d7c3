"""Python binding of libtt_emb.so, the MI355X TT-EmbeddingBag library.

Argument marshalling only: every step of the lookup (planning, forward,
backward, SGD) runs in the library's HIP kernels. PyTorch supplies device
memory and the stream; tensors are passed by data_ptr(). The function names
are those of the C ABI in include/tt_emb.h, whose comments state argument
meaning, layouts, ownership and errors.

If libtt_emb.so has not been built, importing the functions works but the
first call raises TTEmbLibraryMissing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

__all__ = [
    "TTEmbError", "TTEmbLibraryMissing", "TT_OK", "TT_FLAG_BAD_INDEX", "TT_FLAG_BAD_OFFSETS",
    "library_path", "load_library", "make_tables", "tt_emb_workspace_bytes", "tt_emb_plan",
    "tt_emb_forward", "tt_emb_forward_train", "tt_emb_backward", "tt_emb_backward_kept", "tt_emb_backward_sgd",
    "tt_emb_sgd",
    "tt_emb_get_error", "tt_emb_plan_get_view", "tt_emb_plan_counts", "tt_emb_plan_destroy",
    "tt_emb_query_paths", "tt_emb_forward_scratch", "tt_emb_scratch_capacity", "tt_emb_set_timing",
    "tt_emb_kernel_times", "tt_emb_cache_bytes", "tt_emb_cache_build", "tt_emb_plan_cached",
    "tt_emb_forward_cached", "tt_emb_backward_cached", "tt_emb_backward_sgd_cached", "HotCache",
    "TT_PATH_MATRIX_CORE", "TT_PATH_GENERIC", "TT_ERR_STALE", "TT_ERR_SCRATCH", "TT_ERR_CACHE", "Plan",
    "EXPORTS",
]

TT_OK = 0
TT_ERR_INVALID_ARG = -1
TT_ERR_DEVICE_FLAG = -5
TT_ERR_STALE = -6
TT_ERR_SCRATCH = -7
TT_ERR_CACHE = -8
TT_PATH_MATRIX_CORE = 1
TT_PATH_GENERIC = 2
TT_FLAG_BAD_INDEX = 1
TT_FLAG_BAD_OFFSETS = 2

# Every symbol include/tt_emb.h declares.
EXPORTS = (
    "tt_emb_workspace_bytes", "tt_emb_plan", "tt_emb_forward", "tt_emb_forward_train",
    "tt_emb_backward", "tt_emb_backward_kept", "tt_emb_backward_sgd", "tt_emb_sgd",
    "tt_emb_get_error", "tt_emb_plan_get_view", "tt_emb_plan_counts", "tt_emb_plan_destroy",
    "tt_emb_query_paths", "tt_emb_forward_scratch", "tt_emb_scratch_capacity", "tt_emb_set_timing",
    "tt_emb_kernel_times", "tt_emb_cache_bytes", "tt_emb_cache_build", "tt_emb_plan_cached",
    "tt_emb_forward_cached", "tt_emb_backward_cached", "tt_emb_backward_sgd_cached", "tt_emb_status_string",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_lock = threading.Lock()
_lib = None


class TTEmbError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} ({status})")


class TTEmbLibraryMissing(RuntimeError):
    pass


def library_path() -> str:
    """The in-tree libtt_emb.so, or the file TT_EMB_LIBRARY names (an
    instrumented build of the same sources, e.g. with host sanitizers)."""
    return os.environ.get("TT_EMB_LIBRARY") or os.path.join(_HERE, "libtt_emb.so")


class _Table(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int64), ("m", ctypes.c_int32 * 3),
                ("n", ctypes.c_int32 * 3), ("rank", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("g_offset", ctypes.c_int64 * 3)]


class _PathInfo(ctypes.Structure):
    _fields_ = [("forward_path", ctypes.c_int32), ("backward_path", ctypes.c_int32),
                ("keeps_prefix", ctypes.c_int32), ("dg3_by_rows", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)]


class _KernelTime(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("ms", ctypes.c_float)]


class _View(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "key", "i3", "bag_of", "perm", "sorted_i3", "sorted_bag", "group_key", "group_start",
        "chunk_group", "chunk_begin", "chunk_end")] + [
        ("max_groups", ctypes.c_int64), ("max_chunks", ctypes.c_int64)]


def load_library() -> ctypes.CDLL:
    """Load libtt_emb.so from the package directory (no fallback)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise TTEmbLibraryMissing(
                f"{path} is not built; run `python -m tensor_train_compressed_amd.build`")
        lib = ctypes.CDLL(path)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.tt_emb_workspace_bytes.argtypes = [P, i32, i64, i64, i32]
        lib.tt_emb_workspace_bytes.restype = ctypes.c_size_t
        lib.tt_emb_plan.argtypes = [P, i32, P, P, i64, i64, i32, P, ctypes.c_size_t, P,
                                    ctypes.POINTER(P)]
        lib.tt_emb_forward.argtypes = [P, P, P, P, P, P]
        lib.tt_emb_forward_train.argtypes = [P, P, P, P, P, ctypes.POINTER(ctypes.c_uint64), P]
        lib.tt_emb_backward.argtypes = [P, P, P, P, P, P, P, P, P]
        lib.tt_emb_backward_kept.argtypes = [P, ctypes.c_uint64, P, P, P, P, P, P, P, P]
        lib.tt_emb_backward_sgd.argtypes = [P, ctypes.c_uint64, P, P, P, P, ctypes.c_float, P]
        lib.tt_emb_backward_sgd.restype = ctypes.c_int
        lib.tt_emb_query_paths.argtypes = [P, P, P, ctypes.POINTER(_PathInfo)]
        lib.tt_emb_forward_scratch.argtypes = [P, i32, P, P, i64, i64, i32, P, P, P, P, P]
        lib.tt_emb_forward_scratch.restype = ctypes.c_int
        lib.tt_emb_set_timing.argtypes = [P, i32]
        lib.tt_emb_set_timing.restype = ctypes.c_int
        lib.tt_emb_kernel_times.argtypes = [P, ctypes.POINTER(_KernelTime), i32, ctypes.POINTER(i32), P]
        lib.tt_emb_kernel_times.restype = ctypes.c_int
        lib.tt_emb_scratch_capacity.argtypes = []
        lib.tt_emb_scratch_capacity.restype = ctypes.c_size_t
        lib.tt_emb_sgd.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, P]
        lib.tt_emb_get_error.argtypes = [P, ctypes.POINTER(i32), P]
        lib.tt_emb_plan_get_view.argtypes = [P, ctypes.POINTER(_View)]
        lib.tt_emb_plan_counts.argtypes = [P, ctypes.POINTER(i64), ctypes.POINTER(i64), P]
        lib.tt_emb_plan_destroy.argtypes = [P]
        lib.tt_emb_cache_bytes.argtypes = [i64]
        lib.tt_emb_cache_bytes.restype = ctypes.c_size_t
        lib.tt_emb_cache_build.argtypes = [P, P, i64, P, ctypes.c_size_t, P]
        lib.tt_emb_plan_cached.argtypes = [P, i32, P, P, i64, i64, i32, P, i64, P, ctypes.c_size_t, P,
                                           ctypes.POINTER(P)]
        lib.tt_emb_forward_cached.argtypes = [P, P, P, P, P, P, ctypes.POINTER(ctypes.c_uint64), P]
        lib.tt_emb_backward_cached.argtypes = [P, ctypes.c_uint64, P, P, P, P, P, P, P, P, P]
        lib.tt_emb_backward_sgd_cached.argtypes = [P, ctypes.c_uint64, P, P, P, P, P, ctypes.c_float, P]
        lib.tt_emb_status_string.argtypes = [ctypes.c_int]
        lib.tt_emb_status_string.restype = ctypes.c_char_p
        for name in ("tt_emb_plan", "tt_emb_forward", "tt_emb_forward_train", "tt_emb_backward",
                     "tt_emb_backward_kept", "tt_emb_sgd", "tt_emb_get_error", "tt_emb_plan_get_view",
                     "tt_emb_plan_counts", "tt_emb_plan_destroy", "tt_emb_query_paths",
                     "tt_emb_cache_build", "tt_emb_plan_cached", "tt_emb_forward_cached",
                     "tt_emb_backward_cached", "tt_emb_backward_sgd_cached"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def _status_string(status: int) -> str:
    try:
        return load_library().tt_emb_status_string(int(status)).decode()
    except Exception:
        return "status"


def _check(status: int, what: str):
    if status != TT_OK:
        raise TTEmbError(status, what)


def make_tables(tables: Sequence, g_offsets) -> ctypes.Array:
    """C array of tt_emb_table from objects with num_rows, m, n, rank and a
    [T][3] sequence of core element offsets."""
    arr = (_Table * len(tables))()
    for i, t in enumerate(tables):
        arr[i].num_rows = int(t.num_rows)
        for k in range(3):
            arr[i].m[k] = int(t.m[k])
            arr[i].n[k] = int(t.n[k])
            arr[i].g_offset[k] = int(g_offsets[i][k])
        arr[i].rank = int(t.rank)
        arr[i].reserved = 0
    return arr


def _dev_ptr(t, dtype_name: str, what: str, numel: Optional[int] = None,
             at_least: bool = False) -> Optional[int]:
    """data_ptr() of a contiguous device tensor of the given dtype; with
    `numel`, its element count must equal it (or, with at_least, reach it):
    the C ABI takes bare pointers and cannot check extents itself."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if str(t.dtype) != f"torch.{dtype_name}":
        raise ValueError(f"{what} must be {dtype_name}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if numel is not None:
        n = int(t.numel())
        if (n < numel) if at_least else (n != numel):
            raise ValueError(f"{what} has {n} elements, needs {'at least ' if at_least else ''}{numel}")
    return t.data_ptr()


def core_extents(tables_c) -> tuple:
    """Elements of the packed G1, G2, G3 buffers the tables use (the same
    bound applies to the gradient buffers)."""
    ext = [0, 0, 0]
    for t in tables_c:
        n1, n2, n3 = t.n[0], t.n[1], t.n[2]
        R = t.rank
        sizes = (t.m[0] * n1 * R, t.m[1] * R * n2 * R, t.m[2] * R * n3)
        for k in range(3):
            ext[k] = max(ext[k], int(t.g_offset[k]) + sizes[k])
    return tuple(ext)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owns a tt_emb_plan_t; keeps the workspace tensor alive alongside it,
    and the sizes the binding checks tensors against."""

    def __init__(self, handle: int, workspace, L: int, TB: int, D: int, extents=(0, 0, 0)):
        self.handle = handle
        self.workspace = workspace
        self.L, self.TB, self.D = L, TB, D
        self.extents = tuple(extents)

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                load_library().tt_emb_plan_destroy(ctypes.c_void_p(self.handle))
            except Exception:
                pass
            self.handle = None

    def cores(self, g1, g2, g3, names=("g1", "g2", "g3"), dtype="float32"):
        return tuple(_dev_ptr(x, dtype, nm, e, at_least=True)
                     for x, nm, e in zip((g1, g2, g3), names, self.extents))


def tt_emb_workspace_bytes(tables_c, L: int, B: int, chunk: int) -> int:
    return int(load_library().tt_emb_workspace_bytes(tables_c, len(tables_c), L, B, chunk))


def tt_emb_plan(tables_c, indices, offsets, B: int, chunk: int, workspace=None,
                stream=None, cache=None) -> Plan:
    """Plan a batch. `tables_c` from make_tables; indices int64[L] and offsets
    int64[T*B+1] device tensors; workspace a uint8 device tensor (allocated
    here with torch if None); cache a HotCache (tt_emb_plan_cached)."""
    lib = load_library()
    L = int(indices.numel())
    T = len(tables_c)
    need = tt_emb_workspace_bytes(tables_c, L, B, chunk)
    if need == 0:
        raise TTEmbError(-1, "tt_emb_workspace_bytes")
    if workspace is None:
        import torch
        workspace = torch.empty(need, dtype=torch.uint8, device=indices.device)
    h = ctypes.c_void_p()
    args = (tables_c, T, _dev_ptr(indices, "int64", "indices"),
            _dev_ptr(offsets, "int64", "offsets", T * B + 1), L, B, chunk)
    tail = (_dev_ptr(workspace, "uint8", "workspace"), workspace.numel(), _stream(stream), ctypes.byref(h))
    if cache is None:
        _check(lib.tt_emb_plan(*args, *tail), "tt_emb_plan")
    else:
        _check(lib.tt_emb_plan_cached(*args, _dev_ptr(cache.mem, "uint8", "cache"), cache.n_hot, *tail),
               "tt_emb_plan_cached")
    D = int(tables_c[0].n[0] * tables_c[0].n[1] * tables_c[0].n[2])
    pl = Plan(h.value, workspace, L, T * B, D, core_extents(tables_c))
    pl.cache = cache   # kept alive with the plan
    return pl


class HotCache:
    """A hot-row cache's hash table (device memory, owned here) for the
    entries (hot_table[s], hot_row[s]), built on `stream`."""

    def __init__(self, hot_table, hot_row, stream=None):
        import torch
        lib = load_library()
        n = int(hot_row.numel())
        if int(hot_table.numel()) != n:
            raise ValueError("hot_table and hot_row differ in length")
        self.n_hot = n
        nbytes = int(lib.tt_emb_cache_bytes(n))
        if nbytes == 0:
            raise TTEmbError(-2, "tt_emb_cache_bytes")
        self.mem = torch.empty(nbytes, dtype=torch.uint8, device=hot_row.device)
        _check(lib.tt_emb_cache_build(_dev_ptr(hot_table, "int32", "hot_table") if n else None,
                                      _dev_ptr(hot_row, "int64", "hot_row") if n else None, n,
                                      _dev_ptr(self.mem, "uint8", "cache"), nbytes, _stream(stream)),
               "tt_emb_cache_build")


def tt_emb_cache_bytes(n_hot: int) -> int:
    return int(load_library().tt_emb_cache_bytes(int(n_hot)))


def tt_emb_cache_build(hot_table, hot_row, stream=None) -> HotCache:
    return HotCache(hot_table, hot_row, stream)


def tt_emb_plan_cached(tables_c, indices, offsets, B: int, chunk: int, cache: HotCache,
                       workspace=None, stream=None) -> Plan:
    return tt_emb_plan(tables_c, indices, offsets, B, chunk, workspace, stream, cache)


def _hot(plan: Plan, w, what: str):
    if getattr(plan, "cache", None) is None:   # the library refuses the call (TT_ERR_CACHE)
        return _dev_ptr(w, "float32", what)
    n = plan.cache.n_hot
    if n == 0 and w is None:
        return None
    return _dev_ptr(w, "float32", what, n * plan.D)


def tt_emb_forward_cached(plan: Plan, g1, g2, g3, hot_w, out, keep: bool = False, stream=None) -> int:
    """Forward with the hot rows hot_w [n_hot][D]; keep: also keep the
    prefix products (returns their token, else 0)."""
    tok = ctypes.c_uint64(0)
    _check(load_library().tt_emb_forward_cached(
        plan.handle, *plan.cores(g1, g2, g3), _hot(plan, hot_w, "hot_w"),
        _dev_ptr(out, "float32", "out", plan.TB * plan.D), ctypes.byref(tok) if keep else None,
        _stream(stream)), "tt_emb_forward_cached")
    return int(tok.value)


def tt_emb_backward_cached(plan: Plan, kept_token: int, g1, g2, g3, grad_out, dg1, dg2, dg3, hot_dw,
                           stream=None):
    _check(load_library().tt_emb_backward_cached(
        plan.handle, ctypes.c_uint64(int(kept_token)), *plan.cores(g1, g2, g3),
        _dev_ptr(grad_out, "float32", "grad_out", plan.TB * plan.D),
        *plan.cores(dg1, dg2, dg3, ("dg1", "dg2", "dg3")), _hot(plan, hot_dw, "hot_dw"), _stream(stream)),
        "tt_emb_backward_cached")


def tt_emb_backward_sgd_cached(plan: Plan, kept_token: int, g1, g2, g3, hot_w, grad_out, lr: float,
                               stream=None):
    _check(load_library().tt_emb_backward_sgd_cached(
        plan.handle, ctypes.c_uint64(int(kept_token)), *plan.cores(g1, g2, g3), _hot(plan, hot_w, "hot_w"),
        _dev_ptr(grad_out, "float32", "grad_out", plan.TB * plan.D), float(lr), _stream(stream)),
        "tt_emb_backward_sgd_cached")


def tt_emb_forward(plan: Plan, g1, g2, g3, out, stream=None):
    _check(load_library().tt_emb_forward(
        plan.handle, *plan.cores(g1, g2, g3), _dev_ptr(out, "float32", "out", plan.TB * plan.D),
        _stream(stream)), "tt_emb_forward")


def tt_emb_forward_train(plan: Plan, g1, g2, g3, out, stream=None) -> int:
    """Forward that also keeps the prefix products for tt_emb_backward_kept;
    returns the token naming them (0: nothing kept, use tt_emb_backward)."""
    tok = ctypes.c_uint64(0)
    _check(load_library().tt_emb_forward_train(
        plan.handle, *plan.cores(g1, g2, g3), _dev_ptr(out, "float32", "out", plan.TB * plan.D),
        ctypes.byref(tok), _stream(stream)), "tt_emb_forward_train")
    return int(tok.value)


def tt_emb_backward(plan: Plan, g1, g2, g3, grad_out, dg1, dg2, dg3, stream=None):
    _check(load_library().tt_emb_backward(
        plan.handle, *plan.cores(g1, g2, g3),
        _dev_ptr(grad_out, "float32", "grad_out", plan.TB * plan.D),
        *plan.cores(dg1, dg2, dg3, ("dg1", "dg2", "dg3")), _stream(stream)), "tt_emb_backward")


def tt_emb_backward_kept(plan: Plan, kept_token: int, g1, g2, g3, grad_out, dg1, dg2, dg3,
                         stream=None):
    """Backward reusing the prefix products named by kept_token (raises
    TTEmbError with status TT_ERR_STALE when they are not the plan's)."""
    _check(load_library().tt_emb_backward_kept(
        plan.handle, ctypes.c_uint64(int(kept_token)), *plan.cores(g1, g2, g3),
        _dev_ptr(grad_out, "float32", "grad_out", plan.TB * plan.D),
        *plan.cores(dg1, dg2, dg3, ("dg1", "dg2", "dg3")), _stream(stream)), "tt_emb_backward_kept")


def tt_emb_backward_sgd(plan: Plan, kept_token: int, g1, g2, g3, grad_out, lr: float, stream=None):
    """Backward fused with the SGD step: the cores are updated in place on
    the slices the batch touches (kept_token 0: form the prefix products
    again)."""
    _check(load_library().tt_emb_backward_sgd(
        plan.handle, ctypes.c_uint64(int(kept_token)), *plan.cores(g1, g2, g3),
        _dev_ptr(grad_out, "float32", "grad_out", plan.TB * plan.D), float(lr), _stream(stream)),
        "tt_emb_backward_sgd")


def tt_emb_sgd(plan: Plan, g1, g2, g3, dg1, dg2, dg3, lr: float, stream=None):
    _check(load_library().tt_emb_sgd(
        plan.handle, *plan.cores(g1, g2, g3), *plan.cores(dg1, dg2, dg3, ("dg1", "dg2", "dg3")),
        float(lr), _stream(stream)), "tt_emb_sgd")


def tt_emb_query_paths(plan: Plan, g1, g2) -> dict:
    """Which kernels the plan's calls run with these cores (host query)."""
    info = _PathInfo()
    _check(load_library().tt_emb_query_paths(plan.handle, ctypes.c_void_p(g1.data_ptr()),
                                             ctypes.c_void_p(g2.data_ptr()), ctypes.byref(info)),
           "tt_emb_query_paths")
    return {name: int(getattr(info, name)) for name, _ in _PathInfo._fields_}


def tt_emb_set_timing(plan: Optional[Plan], enable: bool = True):
    """Bracket every kernel the plan's calls launch with HIP events (plan
    None: every plan created from now on, its planning kernels included)."""
    _check(load_library().tt_emb_set_timing(None if plan is None else plan.handle, 1 if enable else 0),
           "tt_emb_set_timing")


def tt_emb_kernel_times(plan: Plan, stream=None, max_records: int = 1024) -> list:
    """[(kernel name, ms)] of the launches recorded since the last read, in
    launch order (synchronises the stream)."""
    buf = (_KernelTime * max_records)()
    n = ctypes.c_int32(0)
    _check(load_library().tt_emb_kernel_times(plan.handle, buf, max_records, ctypes.byref(n),
                                              _stream(stream)), "tt_emb_kernel_times")
    return [(buf[i].kernel.decode(), float(buf[i].ms)) for i in range(n.value)]


def tt_emb_scratch_capacity() -> int:
    """Bytes of the library's static scratch buffer (per device)."""
    return int(load_library().tt_emb_scratch_capacity())


def tt_emb_forward_scratch(tables_c, indices, offsets, B: int, chunk: int, g1, g2, g3, out,
                           stream=None):
    """Plan + forward of one batch in the library's static scratch buffer:
    no workspace and no allocation (raises TTEmbError with TT_ERR_SCRATCH
    when the batch does not fit)."""
    T = len(tables_c)
    D = int(tables_c[0].n[0] * tables_c[0].n[1] * tables_c[0].n[2])
    ext = core_extents(tables_c)
    _check(load_library().tt_emb_forward_scratch(
        tables_c, T, _dev_ptr(indices, "int64", "indices"), _dev_ptr(offsets, "int64", "offsets", T * B + 1),
        int(indices.numel()), B, chunk, _dev_ptr(g1, "float32", "g1", ext[0], at_least=True),
        _dev_ptr(g2, "float32", "g2", ext[1], at_least=True), _dev_ptr(g3, "float32", "g3", ext[2], at_least=True),
        _dev_ptr(out, "float32", "out", T * B * D), _stream(stream)), "tt_emb_forward_scratch")


def tt_emb_get_error(plan: Plan, stream=None) -> int:
    """Device error flag (0 or TT_FLAG_* bits); synchronises the stream."""
    f = ctypes.c_int32(0)
    st = load_library().tt_emb_get_error(plan.handle, ctypes.byref(f), _stream(stream))
    if st not in (TT_OK, TT_ERR_DEVICE_FLAG):
        _check(st, "tt_emb_get_error")
    return int(f.value)


def tt_emb_plan_get_view(plan: Plan) -> dict:
    """Device addresses of the planner's int32 tables plus their capacities."""
    v = _View()
    _check(load_library().tt_emb_plan_get_view(plan.handle, ctypes.byref(v)), "tt_emb_plan_get_view")
    return {name: getattr(v, name) for name, _ in _View._fields_}


def tt_emb_plan_counts(plan: Plan, stream=None):
    """(num_groups, num_chunks); synchronises the stream."""
    g, c = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(load_library().tt_emb_plan_counts(plan.handle, ctypes.byref(g), ctypes.byref(c),
                                             _stream(stream)), "tt_emb_plan_counts")
    return int(g.value), int(c.value)


def tt_emb_plan_destroy(plan: Plan):
    if plan.handle:
        _check(load_library().tt_emb_plan_destroy(plan.handle), "tt_emb_plan_destroy")
        plan.handle = None


def plan_table(plan: Plan, name: str, n: int):
    """int32 tensor view (no copy) of one planner table inside the plan's
    workspace tensor; `name` is a tt_emb_plan_view field, `n` its length."""
    addr = tt_emb_plan_get_view(plan)[name]
    off = addr - plan.workspace.data_ptr()
    if off < 0 or off + 4 * n > plan.workspace.numel():
        raise ValueError(f"{name}[{n}] is outside the workspace")
    return plan.workspace[off:off + 4 * n].view(dtype=__import__("torch").int32)
