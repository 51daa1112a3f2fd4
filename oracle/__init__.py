"""Oracle for maximal clique enumeration -- TEST INFRASTRUCTURE ONLY.

A ctypes front for ``mce_oracle.c``, a plain single-threaded CPU Bron-Kerbosch
with Tomita pivoting ("Parallelizing Maximal Clique Enumeration on GPUs",
section 2.3 Algorithm 2 and section 2.4 Algorithm 3). Only the tests, the smoke
check and the bench's CPU-baseline leg may import this package; the GPU library
and its binding never do. It shares no code with them.

Every function here is pinned by tests that do not run the oracle's own
arithmetic again: brute-force subset enumeration, closed-form families, the
worked example of section 2.1, and clique/maximality invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mce_oracle.c")
_LIB = os.path.join(_HERE, "libmce_oracle.so")

GOLDEN = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1

# error classes returned by validate()
OV_ROWPTR, OV_RANGE, OV_LOOP, OV_ORDER, OV_ASYM = 1, 2, 4, 8, 16


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no vector tricks)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        i32p, u64p, i64p = P(ctypes.c_int32), P(ctypes.c_uint64), P(ctypes.c_int64)
        lib.oracle_mix64.argtypes = [ctypes.c_uint64]
        lib.oracle_mix64.restype = ctypes.c_uint64
        lib.oracle_clique_hash.argtypes = [ctypes.c_int, i32p]
        lib.oracle_clique_hash.restype = ctypes.c_uint64
        lib.oracle_validate.argtypes = [ctypes.c_int32, ctypes.c_int64, i32p, i32p]
        lib.oracle_validate.restype = ctypes.c_int
        lib.oracle_peel.argtypes = [ctypes.c_int32, i32p, i32p, i32p, i32p]
        lib.oracle_peel.restype = ctypes.c_int32
        lib.oracle_mce.argtypes = [ctypes.c_int32, i32p, i32p, i32p, i32p, ctypes.c_int32,
                                   ctypes.c_int64, u64p, u64p, u64p, ctypes.c_int32,
                                   i32p, i64p]
        lib.oracle_mce.restype = ctypes.c_int
        lib.oracle_mce_l2.argtypes = [ctypes.c_int32, i32p, i32p, i32p, i32p, ctypes.c_int32,
                                   ctypes.c_int64, u64p, u64p, u64p, ctypes.c_int32,
                                   i32p, i64p]
        lib.oracle_mce_l2.restype = ctypes.c_int
        lib.oracle_mce_each.argtypes = [ctypes.c_int32, i32p, i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int64,
                                        i64p, u64p, u64p, P(ctypes.c_uint8)]
        lib.oracle_mce_each.restype = ctypes.c_int
        lib.oracle_knuth.argtypes = [ctypes.c_int32, i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_uint64, P(ctypes.c_double), i32p]
        lib.oracle_knuth.restype = ctypes.c_int
        lib.oracle_list.argtypes = [ctypes.c_int32, i32p, i32p, i32p, i32p, ctypes.c_int64]
        lib.oracle_list.restype = ctypes.c_int64
        lib.oracle_root_table.argtypes = [ctypes.c_int32, i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, u64p, ctypes.c_int64]
        lib.oracle_root_table.restype = ctypes.c_int64
        _lib = lib
    return _lib


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def mix64(z: int) -> int:
    return int(_load().oracle_mix64(ctypes.c_uint64(z & MASK64)))


def clique_hash(ids) -> int:
    a, p = _i32(ids)
    return int(_load().oracle_clique_hash(len(a), p))


def validate(n: int, row_ptr, col_idx) -> int:
    rp, rpp = _i32(row_ptr)
    ci, cip = _i32(col_idx)
    if rp.shape[0] != n + 1:
        return OV_ROWPTR
    return int(_load().oracle_validate(n, ci.shape[0], rpp, cip))


def peel(n: int, row_ptr, col_idx):
    """Round-synchronous k-core peel. Returns (core, round, d)."""
    rp, rpp = _i32(row_ptr)
    ci, cip = _i32(col_idx)
    core = np.zeros(max(n, 1), np.int32)
    rnd = np.zeros(max(n, 1), np.int32)
    d = _load().oracle_peel(n, rpp, cip, core.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            rnd.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if d < 0:
        raise MemoryError("oracle_peel")
    return core[:n], rnd[:n], int(d)


@dataclass
class Result:
    count: int
    hash: int
    hist: list = field(default_factory=list)   # hist[k] = number of maximal cliques of size k
    nodes: int = 0
    complete: bool = True                     # False if the node budget stopped the search

    def key(self):
        return (self.count, self.hash, tuple(self.hist))


def mce(n: int, row_ptr, col_idx, roots=None, node_budget: int = 0, rnd=None, level: int = 1) -> Result:
    """Maximal cliques of the graph, or of the first-level subtrees of `roots`
    (the cliques whose earliest vertex in the peel order is a listed root).
    level=2 finds the same cliques through second-level subtrees (Algorithm 4)."""
    rp, rpp = _i32(row_ptr)
    ci, cip = _i32(col_idx)
    if rnd is None:
        _, rnd, _ = peel(n, rp, ci)
    rn, rnp = _i32(rnd if n else np.zeros(1, np.int32))
    if roots is None:
        ro, rop, nr = None, None, 0
    else:
        ro, rop = _i32(roots if len(roots) else np.zeros(1, np.int32))
        nr = len(roots)
    maxdeg = int(np.diff(rp).max()) if n else 0
    cap = maxdeg + 3
    hist = np.zeros(cap, np.uint64)
    cnt = ctypes.c_uint64()
    hsh = ctypes.c_uint64()
    hl = ctypes.c_int32()
    nodes = ctypes.c_int64()
    if level not in (1, 2):
        raise ValueError("level is 1 or 2")
    fn = _load().oracle_mce if level == 1 else _load().oracle_mce_l2
    rc = fn(n, rpp, cip, rnp, rop, nr, node_budget, ctypes.byref(cnt),
                            ctypes.byref(hsh),
                            hist.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), cap,
                            ctypes.byref(hl), ctypes.byref(nodes))
    if rc < 0 or rc == 2:
        raise RuntimeError(f"oracle_mce failed with code {rc}")
    return Result(int(cnt.value), int(hsh.value), [int(x) for x in hist[:hl.value]],
                  int(nodes.value), rc == 0)


def list_cliques(n: int, row_ptr, col_idx, rnd=None):
    """All maximal cliques of a small graph as sorted tuples, found by a second,
    list-based (no bitsets) Bron-Kerbosch-Tomita inside the oracle."""
    rp, rpp = _i32(row_ptr)
    ci, cip = _i32(col_idx)
    if rnd is None:
        _, rnd, _ = peel(n, rp, ci)
    rn, rnp = _i32(rnd if n else np.zeros(1, np.int32))
    cap = 1 << 16
    while True:
        out = np.zeros(cap, np.int32)
        got = _load().oracle_list(n, rpp, cip, rnp,
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), cap)
        if got >= 0:
            break
        cap *= 4
    cliques, cur = [], []
    for x in out[:got]:
        if x < 0:
            cliques.append(tuple(cur))
            cur = []
        else:
            cur.append(int(x))
    return cliques


@dataclass
class Estimate:
    walks: int
    nodes: float            # mean of the walks' node estimates
    nodes_se: float         # its standard error
    cliques: float          # mean of the walks' maximal-clique estimates
    cliques_se: float
    max_depth: int          # deepest walk (a clique of max_depth + 1 vertices ends it when maximal)


def knuth(n: int, row_ptr, col_idx, root: int, walks: int, seed: int = 1, rnd=None) -> Estimate:
    """Knuth's random-probe estimate of the first-level subtree of `root`
    (nodes = calls of Algorithm 2, cliques = maximal cliques whose earliest
    vertex is root): unbiased, with the standard error of the mean over walks."""
    rp, rpp = _i32(row_ptr)
    ci, cip = _i32(col_idx)
    if rnd is None:
        _, rnd, _ = peel(n, rp, ci)
    rn, rnp = _i32(rnd)
    sums = (ctypes.c_double * 4)()
    dmax = ctypes.c_int32()
    rc = _load().oracle_knuth(n, rpp, cip, rnp, int(root), int(walks), ctypes.c_uint64(seed & MASK64),
                              sums, ctypes.byref(dmax))
    if rc != 0:
        raise RuntimeError(f"oracle_knuth failed with code {rc}")

    def mean_se(s, s2):
        m = s / walks
        var = max(s2 / walks - m * m, 0.0)
        return m, (var / walks) ** 0.5 if walks > 1 else float("inf")
    nm, nse = mean_se(sums[0], sums[1])
    cm, cse = mean_se(sums[2], sums[3])
    return Estimate(int(walks), nm, nse, cm, cse, int(dmax.value))


def mce_each(n: int, row_ptr, col_idx, roots, root_budget: int, rnd):
    """Each root's first-level subtree on its own node budget: arrays (nodes,
    count, hash, done) in the order of `roots`; count and hash of a root with
    done == 0 are partial."""
    rp, rpp = _i32(row_ptr)
    ci, cip = _i32(col_idx)
    rn, rnp = _i32(rnd)
    ro, rop = _i32(roots if len(roots) else np.zeros(1, np.int32))
    k = len(roots)
    nodes = np.zeros(max(k, 1), np.int64)
    count = np.zeros(max(k, 1), np.uint64)
    hsh = np.zeros(max(k, 1), np.uint64)
    done = np.zeros(max(k, 1), np.uint8)
    rc = _load().oracle_mce_each(n, rpp, cip, rnp, rop, k, int(root_budget),
                                 nodes.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 count.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                 hsh.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                 done.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    if rc != 0:
        raise RuntimeError(f"oracle_mce_each failed with code {rc}")
    return nodes[:k], count[:k], hsh[:k], done[:k]


def root_table(n: int, row_ptr, col_idx, rnd, root: int, W: int, micro: bool, full: bool) -> np.ndarray:
    """One first-level root's bit-encoded induced subgraph (section 2.4 "Induced
    Subgraphs", section 3.4) in the word layout of the engine's table
    inspection: header (|P|, |X|; root, |R| = 1; h(root)), one row of W words
    per member of P (then of X when `full`): bit b set iff the member is
    adjacent to P's b-th member; with `micro`, each P member's neighbours in X
    as a bitset; P's hash terms; the ids of P and X as int32 pairs. P and X in
    ascending id order; adjacency looked up pair by pair in the CSR."""
    rp, rpp = _i32(row_ptr)
    ci, cip = _i32(col_idx)
    rn, rnp = _i32(rnd)
    deg = int(rp[root + 1] - rp[root])
    cap = 3 + (deg * W) + 2 * deg + (deg + 1) // 2 + 4
    out = np.zeros(cap, np.uint64)
    k = _load().oracle_root_table(n, rpp, cip, rnp, int(root), int(W), 1 if micro else 0, 1 if full else 0,
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), cap)
    if k < 0:
        raise ValueError("oracle_root_table: width too small for P, or a bad root")
    return out[:k]
