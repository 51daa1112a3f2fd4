"""Seeded synthetic graph generators shared by the tests, the bench and the oracle checks.

This module only builds input graphs: it holds no part of the clique search itself.
Every generator returns a simple undirected graph in CSR form as two numpy int32
arrays ``(row_ptr, col_idx)``: ``row_ptr`` has n+1 entries, each row of ``col_idx``
is sorted strictly ascending, there are no self-loops and every edge is stored in
both directions (the input form that "Parallelizing Maximal Clique Enumeration on
GPUs", section 3.4, uses for first-level subtrees).

Randomness comes from ``numpy.random.Generator(PCG64(seed))`` so a (generator,
parameters, seed) triple always produces the same bytes.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Graph", "from_edges", "erdos_renyi", "moon_moser", "rmat", "chung_lu",
    "complete", "cycle", "path", "star", "empty", "complete_multipartite",
    "disjoint_union", "relabel", "random_small", "fig1a", "petersen",
    "config_graph", "CONFIGS",
]


@dataclass
class Graph:
    """Undirected simple graph in symmetric CSR form (int32)."""
    n: int
    row_ptr: np.ndarray
    col_idx: np.ndarray
    name: str = ""

    @property
    def nnz(self) -> int:
        return int(self.col_idx.shape[0])

    @property
    def m(self) -> int:
        return self.nnz // 2

    def degrees(self) -> np.ndarray:
        return np.diff(self.row_ptr).astype(np.int64)

    def sha256(self) -> str:
        h = hashlib.sha256()
        h.update(np.int64(self.n).tobytes())
        h.update(np.ascontiguousarray(self.row_ptr, dtype=np.int32).tobytes())
        h.update(np.ascontiguousarray(self.col_idx, dtype=np.int32).tobytes())
        return h.hexdigest()

    def edge_list(self) -> np.ndarray:
        """Edges (u, v) with u < v, shape (m, 2), int64."""
        src = np.repeat(np.arange(self.n, dtype=np.int64), self.degrees())
        dst = self.col_idx.astype(np.int64)
        keep = src < dst
        return np.stack([src[keep], dst[keep]], axis=1)


def from_edges(n: int, u, v, name: str = "") -> Graph:
    """Symmetrise an edge list, drop self-loops and duplicates, return CSR."""
    u = np.asarray(u, dtype=np.int64).ravel()
    v = np.asarray(v, dtype=np.int64).ravel()
    if u.shape != v.shape:
        raise ValueError("u and v must have the same length")
    if n < 0:
        raise ValueError("n must be >= 0")
    if u.size and (u.min() < 0 or v.min() < 0 or u.max() >= n or v.max() >= n):
        raise ValueError("vertex id out of range")
    if n >= 2 ** 31:
        raise ValueError("n must fit int32")
    keep = u != v
    u, v = u[keep], v[keep]
    if n == 0 or u.size == 0:
        return Graph(n, np.zeros(n + 1, np.int32), np.zeros(0, np.int32), name)
    # undirected, deduplicated, sorted by (lo, hi)
    key = np.minimum(u, v) * n + np.maximum(u, v)
    del u, v
    key.sort()
    if key.size > 1:
        key = key[np.concatenate(([True], key[1:] != key[:-1]))]
    lo, hi = np.divmod(key, n)
    del key
    m = lo.size
    if 2 * m >= 2 ** 31:
        raise ValueError("nnz must fit int32")
    # row v = its smaller neighbours (ascending), then its larger ones (ascending)
    cnt_up = np.bincount(lo, minlength=n)
    cnt_dn = np.bincount(hi, minlength=n)
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(cnt_up + cnt_dn, out=row_ptr[1:])
    dst = np.empty(2 * m, dtype=np.int32)
    # larger neighbours: the (lo, hi) order already groups them by lo, ascending
    up_start = np.cumsum(cnt_up) - cnt_up
    dst[row_ptr[:-1][lo] + cnt_dn[lo] + (np.arange(m, dtype=np.int64) - up_start[lo])] = hi
    # smaller neighbours: group by hi, ascending lo
    rkey = hi * n + lo
    del lo
    rkey.sort()
    rhi, rlo = np.divmod(rkey, n)
    del rkey
    dn_start = np.cumsum(cnt_dn) - cnt_dn
    dst[row_ptr[:-1][rhi] + (np.arange(m, dtype=np.int64) - dn_start[rhi])] = rlo
    return Graph(n, row_ptr.astype(np.int32), dst, name)


# ---------------------------------------------------------------- small families
def empty(n: int) -> Graph:
    return from_edges(n, [], [], f"empty{n}")


def complete(n: int) -> Graph:
    iu, ju = np.triu_indices(n, 1)
    return from_edges(n, iu, ju, f"K{n}")


def cycle(n: int) -> Graph:
    i = np.arange(n)
    return from_edges(n, i, (i + 1) % n, f"C{n}")


def path(n: int) -> Graph:
    i = np.arange(max(n - 1, 0))
    return from_edges(n, i, i + 1, f"P{n}")


def star(leaves: int) -> Graph:
    return from_edges(leaves + 1, np.zeros(leaves, np.int64), np.arange(1, leaves + 1), f"star{leaves}")


def complete_multipartite(sizes) -> Graph:
    """Complement of disjoint cliques: vertices in different parts are adjacent."""
    sizes = [int(s) for s in sizes]
    part = np.repeat(np.arange(len(sizes)), sizes)
    n = part.size
    iu, ju = np.triu_indices(n, 1)
    keep = part[iu] != part[ju]
    return from_edges(n, iu[keep], ju[keep], "K(" + ",".join(map(str, sizes)) + ")")


def moon_moser(n: int) -> Graph:
    """Moon-Moser graph on n = 3k vertices: i ~ j iff i//3 != j//3."""
    if n % 3:
        raise ValueError("Moon-Moser needs n divisible by 3")
    g = complete_multipartite([3] * (n // 3))
    g.name = f"moon_moser{n}"
    return g


def petersen() -> Graph:
    outer = [(i, (i + 1) % 5) for i in range(5)]
    inner = [(5 + i, 5 + (i + 2) % 5) for i in range(5)]
    spokes = [(i, i + 5) for i in range(5)]
    e = np.array(outer + inner + spokes)
    return from_edges(10, e[:, 0], e[:, 1], "petersen")


def fig1a() -> Graph:
    """Six vertices A..F (ids 0..5) whose only maximal cliques are ABCD and AEF."""
    A, B, C, D, E, F = range(6)
    edges = [(A, B), (A, C), (A, D), (B, C), (B, D), (C, D), (A, E), (A, F), (E, F)]
    e = np.array(edges)
    return from_edges(6, e[:, 0], e[:, 1], "fig1a")


def disjoint_union(*gs: Graph) -> Graph:
    us, vs, off = [], [], 0
    for g in gs:
        el = g.edge_list()
        us.append(el[:, 0] + off)
        vs.append(el[:, 1] + off)
        off += g.n
    u = np.concatenate(us) if us else np.zeros(0, np.int64)
    v = np.concatenate(vs) if vs else np.zeros(0, np.int64)
    return from_edges(off, u, v, "+".join(g.name for g in gs))


def relabel(g: Graph, perm) -> Graph:
    """Vertex v of g becomes perm[v]."""
    perm = np.asarray(perm, dtype=np.int64)
    el = g.edge_list()
    return from_edges(g.n, perm[el[:, 0]], perm[el[:, 1]], g.name + "~relabel")


def random_small(n: int, p: float, seed: int) -> Graph:
    """G(n, p) by one Bernoulli draw per vertex pair (for small n)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    iu, ju = np.triu_indices(n, 1)
    keep = rng.random(iu.size) < p
    return from_edges(n, iu[keep], ju[keep], f"gnp{n}_{p}_{seed}")


def hub_clique(core: int, hubs: int, leaves: int, frac: float, missing: int, seed: int) -> Graph:
    """A near-clique with hubs: `core` vertices pairwise adjacent except for
    `missing` random pairs; each of `hubs` hubs is adjacent to a random `frac` of
    the core and to `leaves` leaves of its own. The leaves peel first and the hubs
    before the core, so every core root's X holds hubs whose CSR rows are far
    longer than its P. Ids are shuffled."""
    rng = np.random.Generator(np.random.PCG64(seed))
    iu, ju = np.triu_indices(core, 1)
    keep = np.ones(iu.size, bool)
    keep[rng.choice(iu.size, size=min(missing, iu.size), replace=False)] = False
    us, vs = [iu[keep]], [ju[keep]]
    nxt = core + hubs
    for h in range(hubs):
        nb = np.flatnonzero(rng.random(core) < frac)
        us.append(np.full(nb.size, core + h))
        vs.append(nb)
        us.append(np.full(leaves, core + h))
        vs.append(np.arange(nxt, nxt + leaves))
        nxt += leaves
    perm = rng.permutation(nxt)
    u = perm[np.concatenate(us).astype(np.int64)]
    v = perm[np.concatenate(vs).astype(np.int64)]
    return from_edges(nxt, u, v, f"hubclique{core}_{hubs}_{leaves}_{seed}")


# ---------------------------------------------------------------- benchmark families
def erdos_renyi(n: int, p: float, seed: int) -> Graph:
    """G(n, p): every pair i<j independently with probability p.

    Rows are drawn in blocks: block rows [r0, r1) draw a (r1-r0) x n array of
    uniforms and keep the strict upper triangle, so each pair gets exactly one
    Bernoulli(p) draw.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    us, vs = [], []
    block = max(1, (1 << 22) // max(n, 1))
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        draw = rng.random((r1 - r0, n)) < p
        rows = np.arange(r0, r1)[:, None]
        draw &= np.arange(n)[None, :] > rows
        ii, jj = np.nonzero(draw)
        us.append(ii + r0)
        vs.append(jj)
    u = np.concatenate(us) if us else np.zeros(0, np.int64)
    v = np.concatenate(vs) if vs else np.zeros(0, np.int64)
    return from_edges(n, u, v, f"er{n}_{p}_{seed}")


def rmat(scale: int, edge_factor: int, a: float, b: float, c: float, d: float, seed: int) -> Graph:
    """R-MAT: edge_factor * 2^scale samples; each level picks a quadrant with
    probabilities (a, b, c, d). No noise and no label permutation. The samples are
    then symmetrised, self-loops and duplicates dropped."""
    if abs(a + b + c + d - 1.0) > 1e-9:
        raise ValueError("R-MAT probabilities must sum to 1")
    rng = np.random.Generator(np.random.PCG64(seed))
    n = 1 << scale
    m = edge_factor * n
    idt = np.int32 if scale < 31 else np.int64
    u = np.zeros(m, dtype=idt)
    v = np.zeros(m, dtype=idt)
    # buffers reused across levels (fresh large temporaries cost page faults)
    r = np.empty(m, dtype=np.float64)
    q = np.empty(m, dtype=np.int8)
    t = np.empty(m, dtype=np.bool_)
    c0, c1, c2 = a, a + b, a + b + c
    for _ in range(scale):
        rng.random(out=r)
        # quadrant 0:(0,0) 1:(0,1) 2:(1,0) 3:(1,1) = the number of cut points <= r
        np.greater_equal(r, c0, out=t)
        q[:] = t
        np.greater_equal(r, c1, out=t)
        q += t
        np.greater_equal(r, c2, out=t)
        q += t
        u <<= 1
        u |= q >> 1
        v <<= 1
        v |= q & 1
    return from_edges(n, u, v, f"rmat{scale}_{edge_factor}_{seed}")


def _chung_lu_weights(n: int, mean: float, gamma: float, w_max: float) -> np.ndarray:
    """w_i = c (i + i0)^(-1/(gamma-1)), with w_0 = w_max and mean(w) = mean."""
    alpha = 1.0 / (gamma - 1.0)
    i = np.arange(n, dtype=np.float64)

    def mean_of(i0):
        c = w_max * i0 ** alpha
        return float(np.mean(c * (i + i0) ** (-alpha)))

    lo, hi = 1e-9, 1e12
    for _ in range(200):
        mid = math.sqrt(lo * hi)
        nlo, nhi = (mid, hi) if mean_of(mid) < mean else (lo, mid)
        if (nlo, nhi) == (lo, hi):
            break   # a fixed point: every further step would leave (lo, hi) as they are
        lo, hi = nlo, nhi
    i0 = math.sqrt(lo * hi)
    return w_max * i0 ** alpha * (i + i0) ** (-alpha)


def chung_lu(n: int, mean: float, gamma: float, w_max: float | None, seed: int,
             planted: int = 0, planted_min: int = 20, planted_max: int = 60) -> Graph:
    """Chung-Lu graph: pair (i, j) is an edge with probability min(1, w_i w_j / sum w).

    Sampled exactly by per-row geometric skipping over the descending weights
    (Miller and Hagberg, 2011), vectorised across rows. Optionally adds `planted`
    cliques whose sizes are uniform on [planted_min, planted_max] and whose members
    are drawn uniformly without replacement.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if w_max is None:
        w_max = math.sqrt(n * mean)
    w = _chung_lu_weights(n, mean, gamma, w_max)
    S = float(w.sum())
    us, vs = [], []
    U = np.arange(n - 1, dtype=np.int64)
    V = U + 1
    P = np.minimum(w[U] * w[V] / S, 1.0)
    while U.size:
        need_skip = P < 1.0
        r = 1.0 - rng.random(U.size)
        with np.errstate(divide="ignore"):
            skip = np.where(need_skip, np.floor(np.log(r) / np.log1p(-np.minimum(P, 1.0 - 1e-16))), 0.0)
        skip = np.minimum(skip, float(n))
        V = V + skip.astype(np.int64)
        alive = V < n
        U, V, P = U[alive], V[alive], P[alive]
        if not U.size:
            break
        Q = np.minimum(w[U] * w[V] / S, 1.0)
        r2 = rng.random(U.size)
        acc = r2 < Q / P
        us.append(U[acc])
        vs.append(V[acc])
        P = Q
        V = V + 1
        alive = (V < n) & (P > 0)
        U, V, P = U[alive], V[alive], P[alive]
    for _ in range(planted):
        s = int(rng.integers(planted_min, planted_max + 1))
        mem = rng.choice(n, size=s, replace=False)
        iu, ju = np.triu_indices(s, 1)
        us.append(mem[iu].astype(np.int64))
        vs.append(mem[ju].astype(np.int64))
    u = np.concatenate(us) if us else np.zeros(0, np.int64)
    v = np.concatenate(vs) if vs else np.zeros(0, np.int64)
    return from_edges(n, u, v, f"chung_lu{n}_{mean}_{gamma}_{seed}")


# ---------------------------------------------------------------- the five workloads
CONFIGS = {
    0: "Erdos-Renyi G(2000, 0.01)",
    1: "Moon-Moser n=45 (complement of 15 disjoint triangles)",
    2: "R-MAT scale 20, edge factor 16, (a,b,c,d)=(0.57,0.19,0.19,0.05)",
    3: "Chung-Lu n=500k, mean degree 30, exponent 2.3, +2000 planted cliques of size 20..60",
    4: "Chung-Lu n=4M, mean degree 50 (~100M edges), exponent 2.1, max expected degree 20000",
}


def config_graph(idx: int, seed: int = 1) -> Graph:
    if idx == 0:
        g = erdos_renyi(2000, 0.01, seed)
    elif idx == 1:
        g = moon_moser(45)
    elif idx == 2:
        g = rmat(20, 16, 0.57, 0.19, 0.19, 0.05, seed)
    elif idx == 3:
        g = chung_lu(500_000, 30.0, 2.3, None, seed, planted=2000)
    elif idx == 4:
        g = chung_lu(4_000_000, 50.0, 2.1, 20000.0, seed)
    else:
        raise ValueError(f"no config {idx}")
    g.name = f"cfg{idx}:" + CONFIGS[idx]
    return g
