"""Python binding of the MI355X maximal clique enumeration engine (libmce.so).

The functions named ``mce_*`` mirror the C ABI in ``include/mce.h`` one to one and
only marshal arguments; every step of the computation runs in the HIP library.
``Engine`` is a thin convenience wrapper that takes torch tensors (device memory
and streams come from PyTorch; nothing else does).

If the library has not been built, importing still works but every call raises
``MceLibraryMissing``: there is no CPU fallback.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import weakref
from dataclasses import dataclass, field

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmce.so")

MCE_OK, MCE_ERR_ARG, MCE_ERR_GRAPH, MCE_ERR_NOMEM = 0, -1, -2, -3
MCE_ERR_DEVICE, MCE_ERR_STATE, MCE_ERR_TIMEOUT, MCE_ERR_LIMIT = -4, -5, -6, -7
MCE_GRAPH_ROWPTR, MCE_GRAPH_RANGE, MCE_GRAPH_LOOP, MCE_GRAPH_ORDER, MCE_GRAPH_ASYM = 1, 2, 4, 8, 16
MCE_FLAG_HBM_STAGING, MCE_FLAG_PHASE_TIMES, MCE_FLAG_COUNTERS, MCE_FLAG_NO_MICRO, MCE_FLAG_L2 = 1, 2, 4, 8, 16
MCE_FLAG_SEARCH_TIMES = 32
MCE_FLAG_SERIAL = 64
MCE_SUBGRAPH_AUTO, MCE_SUBGRAPH_PARTIAL, MCE_SUBGRAPH_FULL = 0, 1, 2

# every function the C header declares
EXPORTS = ("mce_config_init", "mce_create", "mce_run", "mce_run_roots", "mce_run_static", "mce_result",
           "mce_graph_info", "mce_ordering", "mce_root_table", "mce_stats", "mce_worker_trace",
           "mce_last_error", "mce_status_string", "mce_destroy")


class MceLibraryMissing(RuntimeError):
    pass


class MceError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status
        self.message = message


class mce_config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("device", ctypes.c_int32),
                ("worker_list", ctypes.c_int32), ("donate_min_p", ctypes.c_int32),
                ("validate", ctypes.c_int32), ("max_workers", ctypes.c_int32),
                ("timeout_ms", ctypes.c_int64), ("flags", ctypes.c_uint32),
                ("subgraph", ctypes.c_int32), ("micro_donate_min_p", ctypes.c_int32),
                ("micro_stack_frames", ctypes.c_int32)]


class mce_graph_facts(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("nnz", ctypes.c_int64), ("max_degree", ctypes.c_int32),
                ("degeneracy", ctypes.c_int32), ("rounds", ctypes.c_int32),
                ("max_p", ctypes.c_int32), ("max_x", ctypes.c_int32),
                ("isolated", ctypes.c_int64), ("roots", ctypes.c_int64),
                ("graph_errors", ctypes.c_uint32), ("subgraph", ctypes.c_int32), ("level", ctypes.c_int32),
                ("complete", ctypes.c_int32), ("roots_started", ctypes.c_int64)]


class mce_worker_record(ctypes.Structure):
    _fields_ = [("launch", ctypes.c_int32), ("worker", ctypes.c_int32),
                ("start_tick", ctypes.c_uint64), ("first_tick", ctypes.c_uint64),
                ("last_tick", ctypes.c_uint64), ("end_tick", ctypes.c_uint64),
                ("busy_ticks", ctypes.c_uint64), ("nodes", ctypes.c_uint64),
                ("donations", ctypes.c_uint64), ("received", ctypes.c_uint64),
                ("hw_location", ctypes.c_uint64), ("leaves", ctypes.c_uint64),
                ("pivot_words", ctypes.c_uint64), ("branches", ctypes.c_uint64),
                ("xx_tests", ctypes.c_uint64)]


class mce_run_stats(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("workers", ctypes.c_int32),
                ("launches", ctypes.c_int32), ("handover_round", ctypes.c_int32),
                ("nodes", ctypes.c_uint64), ("leaves", ctypes.c_uint64),
                ("donations", ctypes.c_uint64), ("pivot_rows", ctypes.c_uint64),
                ("pivot_words", ctypes.c_uint64), ("xx_tests", ctypes.c_uint64),
                ("table_words", ctypes.c_uint64), ("busy_ticks", ctypes.c_uint64),
                ("max_busy_ticks", ctypes.c_uint64), ("max_nodes", ctypes.c_uint64),
                ("kernel_ticks", ctypes.c_uint64), ("tick_hz", ctypes.c_double),
                ("ms_total", ctypes.c_double), ("ms_validate", ctypes.c_double),
                ("ms_peel", ctypes.c_double), ("ms_orient", ctypes.c_double),
                ("ms_search", ctypes.c_double), ("ms_build", ctypes.c_double),
                ("donate_ticks", ctypes.c_uint64), ("setup_ticks", ctypes.c_uint64),
                ("first_ticks", ctypes.c_uint64), ("start_spread_ticks", ctypes.c_uint64),
                ("claim_checks", ctypes.c_uint64), ("donate_ok_ticks", ctypes.c_uint64),
                ("branches", ctypes.c_uint64),
                ("max_stack_frames", ctypes.c_uint64),
                ("micro_roots", ctypes.c_int32),
                ("micro_stack_cap", ctypes.c_int32),
                ("steps", ctypes.c_uint64),
                ("lane_steps", ctypes.c_uint64),
                ("peel_ticks", ctypes.c_uint64 * 4),
                ("launch_sub", ctypes.c_int32 * 16),
                ("launch_roots", ctypes.c_int32 * 16),
                ("launch_build_ms", ctypes.c_float * 16),
                ("launch_search_ms", ctypes.c_float * 16),
                ("launch_words", ctypes.c_uint64 * 16),
                ("act_cycles", ctypes.c_uint64 * 7)]

# Activities of mce_run_stats.act_cycles, in order.
ACTIVITIES = ("worker_list", "idle", "task_start", "pivot", "set_ops", "stack", "cliques")


_lib = None


def lib_built() -> bool:
    return os.path.exists(LIB_PATH)


def load_library():
    """Load libmce.so; raises MceLibraryMissing if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MceLibraryMissing(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                                "python -m maximal_clique_enumeration_amd.build")
    # torch first: the library then binds to the HIP runtime torch loaded. Loaded
    # the other way round, the process holds two HIP runtimes, and the one the
    # library uses may find no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    P = ctypes.POINTER
    lib.mce_config_init.argtypes = [P(mce_config)]
    lib.mce_create.argtypes = [P(mce_config), P(vp)]
    lib.mce_run.argtypes = [vp, i32, i64, vp, vp, vp]
    lib.mce_run_roots.argtypes = [vp, i32, i64, vp, vp, vp, i32, vp]
    lib.mce_run_static.argtypes = [vp, i32, i64, vp, vp, vp]
    lib.mce_result.argtypes = [vp, P(ctypes.c_uint64), P(ctypes.c_uint64), P(ctypes.c_uint64), i32, P(i32)]
    lib.mce_graph_info.argtypes = [vp, P(mce_graph_facts)]
    lib.mce_ordering.argtypes = [vp, vp, vp, vp]
    lib.mce_root_table.argtypes = [vp, i32, P(ctypes.c_uint64), i64, P(i64), P(i32), vp]
    lib.mce_stats.argtypes = [vp, P(mce_run_stats)]
    lib.mce_worker_trace.argtypes = [vp, P(mce_worker_record), i32, P(i32)]
    lib.mce_last_error.argtypes = [vp]
    lib.mce_last_error.restype = ctypes.c_char_p
    lib.mce_status_string.argtypes = [ctypes.c_int]
    lib.mce_status_string.restype = ctypes.c_char_p
    lib.mce_destroy.argtypes = [vp]
    lib.mce_destroy.restype = None
    for name in ("mce_config_init", "mce_create", "mce_run", "mce_run_roots", "mce_run_static", "mce_result",
                 "mce_graph_info", "mce_ordering", "mce_root_table", "mce_stats"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


# ---------------------------------------------------------------- C ABI mirrors
def mce_config_init(cfg: mce_config) -> int:
    return load_library().mce_config_init(ctypes.byref(cfg))


def mce_create(cfg: mce_config | None, out: ctypes.c_void_p) -> int:
    return load_library().mce_create(ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(out))


def mce_run(engine, n, nnz, row_ptr, col_idx, stream) -> int:
    return load_library().mce_run(engine, n, nnz, row_ptr, col_idx, stream)


def mce_run_roots(engine, n, nnz, row_ptr, col_idx, roots, nroots, stream) -> int:
    return load_library().mce_run_roots(engine, n, nnz, row_ptr, col_idx, roots, nroots, stream)


def mce_run_static(engine, n, nnz, row_ptr, col_idx, stream) -> int:
    return load_library().mce_run_static(engine, n, nnz, row_ptr, col_idx, stream)


def mce_result(engine, count, hash_, hist, hist_cap, hist_len) -> int:
    return load_library().mce_result(engine, count, hash_, hist, hist_cap, hist_len)


def mce_graph_info(engine, info: mce_graph_facts) -> int:
    return load_library().mce_graph_info(engine, ctypes.byref(info))


def mce_ordering(engine, core, round_, stream) -> int:
    return load_library().mce_ordering(engine, core, round_, stream)


def mce_root_table(engine, root, words, cap, length, form, stream) -> int:
    return load_library().mce_root_table(engine, root, words, cap, length, form, stream)


def mce_stats(engine, stats: mce_run_stats) -> int:
    return load_library().mce_stats(engine, ctypes.byref(stats))


def mce_worker_trace(engine, out, cap: int, count) -> int:
    return load_library().mce_worker_trace(engine, out, cap, count)


def mce_last_error(engine) -> str:
    return load_library().mce_last_error(engine).decode()


def mce_status_string(status: int) -> str:
    return load_library().mce_status_string(status).decode()


def mce_destroy(engine) -> None:
    load_library().mce_destroy(engine)


def status_name(status: int) -> str:
    names = {0: "MCE_OK", -1: "MCE_ERR_ARG", -2: "MCE_ERR_GRAPH", -3: "MCE_ERR_NOMEM",
             -4: "MCE_ERR_DEVICE", -5: "MCE_ERR_STATE", -6: "MCE_ERR_TIMEOUT", -7: "MCE_ERR_LIMIT"}
    return names.get(status, f"status {status}")


# ---------------------------------------------------------------- torch wrapper
@dataclass
class Result:
    count: int
    hash: int
    hist: list = field(default_factory=list)
    complete: bool = True   # False: the search stopped at the time limit and these are partial sums

    def key(self):
        return (self.count, self.hash, tuple(self.hist))


# Engines still open when the interpreter exits are destroyed here, while the
# HIP runtime (and a profiler attached to it) is still up: device memory freed
# from a finaliser that runs after the runtime's own teardown can crash the exit.
_live = weakref.WeakSet()


@atexit.register
def _close_all():
    for e in list(_live):
        try:
            e.close()
        except Exception:
            pass


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else ctypes.c_void_p(0)


class Engine:
    """One engine on one GPU. Inputs are int32 CUDA tensors (CSR)."""

    def __init__(self, device: int | None = None, worker_list: bool = True, donate_min_p: int = 1,
                 validate: bool = True, max_workers: int = 0, timeout_ms: int = 120000,
                 hbm_staging: bool = False, phase_times: bool = False, subgraph: str = "auto",
                 counters: bool = False, micro: bool = True, micro_donate_min_p: int = 10, level: int = 1,
                 search_times: bool = False, overlap: bool = True, micro_stack_frames: int = 0):
        import torch
        if device is None:
            device = torch.cuda.current_device()
        self.device = device
        cfg = mce_config()
        self._check(mce_config_init(cfg), "mce_config_init", None)
        cfg.device = device
        cfg.worker_list = 1 if worker_list else 0
        cfg.donate_min_p = donate_min_p
        cfg.micro_donate_min_p = micro_donate_min_p
        cfg.micro_stack_frames = micro_stack_frames
        cfg.validate = 1 if validate else 0
        cfg.max_workers = max_workers
        cfg.timeout_ms = timeout_ms
        if level not in (1, 2):
            raise ValueError("level is 1 (first-level subtrees) or 2 (second-level subtrees)")
        cfg.flags = ((MCE_FLAG_HBM_STAGING if hbm_staging else 0) | (MCE_FLAG_PHASE_TIMES if phase_times else 0)
                     | (MCE_FLAG_COUNTERS if counters else 0) | (0 if micro else MCE_FLAG_NO_MICRO)
                     | (MCE_FLAG_L2 if level == 2 else 0) | (MCE_FLAG_SEARCH_TIMES if search_times else 0)
                     | (0 if overlap else MCE_FLAG_SERIAL))
        modes = {"auto": MCE_SUBGRAPH_AUTO, "partial": MCE_SUBGRAPH_PARTIAL, "full": MCE_SUBGRAPH_FULL}
        if subgraph not in modes:
            raise ValueError(f"subgraph must be one of {sorted(modes)}")
        cfg.subgraph = modes[subgraph]
        h = ctypes.c_void_p()
        with torch.cuda.device(device):
            self._check(mce_create(cfg, h), "mce_create", None)
        self._h = h
        _live.add(self)

    def _check(self, status, what, handle):
        if status != MCE_OK:
            msg = mce_last_error(handle) if handle else what
            raise MceError(status, msg)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            mce_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    @staticmethod
    def _check_csr(row_ptr, col_idx):
        import torch
        for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
            if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int32 CUDA tensor")

    def run_static(self, row_ptr, col_idx, stream=None) -> Result:
        """mce_run_static: the whole graph, every device buffer carved from the
        library's static scratch (no allocation)."""
        import torch
        self._check_csr(row_ptr, col_idx)
        if stream is None:
            stream = torch.cuda.current_stream(row_ptr.device)
        st = mce_run_static(self._h, row_ptr.numel() - 1, col_idx.numel(), _ptr(row_ptr), _ptr(col_idx),
                            ctypes.c_void_p(stream.cuda_stream))
        self._check(st, "mce_run_static", self._h)
        return self.result()

    def run(self, row_ptr, col_idx, roots=None, stream=None, partial_ok: bool = False) -> Result:
        """Enumerate all maximal cliques (or those of the first-level subtrees of
        `roots`). Returns (count, hash, hist). With partial_ok, a search stopped at
        the time limit returns the cliques found before it (complete=False)
        instead of raising."""
        import torch
        self._check_csr(row_ptr, col_idx)
        n = row_ptr.numel() - 1
        nnz = col_idx.numel()
        if stream is None:
            stream = torch.cuda.current_stream(row_ptr.device)
        sp = ctypes.c_void_p(stream.cuda_stream)
        if roots is None:
            st = mce_run(self._h, n, nnz, _ptr(row_ptr), _ptr(col_idx), sp)
        else:
            if roots.dtype != torch.int32 or not roots.is_cuda or not roots.is_contiguous():
                raise ValueError("roots must be a contiguous int32 CUDA tensor")
            st = mce_run_roots(self._h, n, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(roots), roots.numel(), sp)
        if not (partial_ok and st == MCE_ERR_TIMEOUT and self.graph_info()["roots_started"] > 0):
            self._check(st, "mce_run", self._h)
        return self.result()

    def result(self) -> Result:
        """Results of the last run; complete=False after a search stopped at the time limit."""
        cnt = ctypes.c_uint64()
        hsh = ctypes.c_uint64()
        hl = ctypes.c_int32()
        st = mce_result(self._h, ctypes.byref(cnt), ctypes.byref(hsh), None, 0, ctypes.byref(hl))
        if st != MCE_ERR_TIMEOUT:
            self._check(st, "mce_result", self._h)
        cap = max(hl.value, 1)
        buf = (ctypes.c_uint64 * cap)()
        st2 = mce_result(self._h, None, None, buf, cap, ctypes.byref(hl))
        if st2 != MCE_ERR_TIMEOUT:
            self._check(st2, "mce_result", self._h)
        return Result(int(cnt.value), int(hsh.value), [int(buf[i]) for i in range(hl.value)], st == MCE_OK)

    def graph_info(self) -> dict:
        info = mce_graph_facts()
        self._check(mce_graph_info(self._h, info), "mce_graph_info", self._h)
        return {name: getattr(info, name) for name, _ in mce_graph_facts._fields_}

    def ordering(self, n: int, device=None):
        """(core, round) of the last run as int32 CUDA tensors."""
        import torch
        dev = torch.device("cuda", self.device if device is None else device)
        core = torch.empty(n, dtype=torch.int32, device=dev)
        rnd = torch.empty(n, dtype=torch.int32, device=dev)
        stream = torch.cuda.current_stream(dev)
        self._check(mce_ordering(self._h, _ptr(core), _ptr(rnd), ctypes.c_void_p(stream.cuda_stream)),
                    "mce_ordering", self._h)
        return core, rnd

    def root_table(self, root: int):
        """(words as a uint64 numpy array, form) of the table the last run built
        for first-level root `root`, or None when it built none (see mce.h)."""
        import numpy as np
        import torch
        stream = ctypes.c_void_p(torch.cuda.current_stream(torch.device("cuda", self.device)).cuda_stream)
        length = ctypes.c_int64()
        form = ctypes.c_int32()
        st = mce_root_table(self._h, int(root), None, 0, ctypes.byref(length), ctypes.byref(form), stream)
        if st == MCE_ERR_STATE:
            return None
        if st not in (MCE_OK, MCE_ERR_ARG):
            self._check(st, "mce_root_table", self._h)
        words = np.zeros(max(1, length.value), np.uint64)
        self._check(mce_root_table(self._h, int(root), words.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                   length.value, ctypes.byref(length), ctypes.byref(form), stream),
                    "mce_root_table", self._h)
        return words[:length.value], form.value

    def worker_trace(self) -> list[dict]:
        """One record per wavefront of the last run's search launches."""
        n = ctypes.c_int32()
        self._check(mce_worker_trace(self._h, None, 0, ctypes.byref(n)), "mce_worker_trace", self._h)
        recs = (mce_worker_record * max(1, n.value))()
        self._check(mce_worker_trace(self._h, recs, n.value, ctypes.byref(n)), "mce_worker_trace", self._h)
        return [{name: getattr(r, name) for name, _ in mce_worker_record._fields_} for r in recs[:n.value]]

    def stats(self) -> dict:
        st = mce_run_stats()
        st.struct_size = ctypes.sizeof(mce_run_stats)
        self._check(mce_stats(self._h, st), "mce_stats", self._h)
        out = {name: getattr(st, name) for name, _ in mce_run_stats._fields_}
        for key in ("peel_ticks", "launch_sub", "launch_roots", "launch_build_ms", "launch_search_ms",
                    "launch_words"):
            out[key] = list(out[key])[: (4 if key == "peel_ticks" else out["launches"])]
        out["act_cycles"] = dict(zip(ACTIVITIES, list(out["act_cycles"])))
        return out
