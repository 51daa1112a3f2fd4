"""Independent checkers for the oracle: brute-force subset enumeration and a
second implementation of the clique-set hash in Python integers.

Nothing here calls the oracle; it only reads a graph in CSR form.
"""
import numpy as np

M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def mix64(z):
    """SplitMix64 finaliser (Steele, Lea and Flood, OOPSLA 2014) on Python ints."""
    z &= M64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & M64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & M64
    z ^= z >> 31
    return z


def clique_hash(clique):
    s = 0
    for c in clique:
        s = (s + mix64(int(c) + GOLDEN)) & M64
    return mix64(s + len(clique) * GOLDEN)


def set_summary(cliques):
    """(count, hash, hist) of a collection of cliques, hist indexed by size."""
    cliques = list(cliques)
    h = 0
    k = max((len(c) for c in cliques), default=-1)
    hist = [0] * (k + 1)
    for c in cliques:
        h = (h + clique_hash(c)) & M64
        hist[len(c)] += 1
    return len(cliques), h, hist


def adjacency_masks(n, row_ptr, col_idx):
    adj = [0] * n
    for v in range(n):
        for e in range(row_ptr[v], row_ptr[v + 1]):
            adj[v] |= 1 << int(col_idx[e])
    return adj


def brute_maximal_cliques(n, row_ptr, col_idx):
    """Every maximal clique of a graph with n <= 22 vertices, by testing all 2^n
    vertex subsets: S is a clique iff each member is adjacent to all others, and
    maximal iff no outside vertex is adjacent to all of S (section 2.1)."""
    assert n <= 22
    if n == 0:
        return []
    adj = np.array(adjacency_masks(n, row_ptr, col_idx), dtype=np.int64)
    N = 1 << n
    S = np.arange(N, dtype=np.int64)
    clique = np.zeros(N, dtype=bool)
    clique[0] = True
    for b in range(n):                      # subsets whose highest member is b
        lo, hi = 1 << b, 1 << (b + 1)
        rest = S[lo:hi] - lo
        clique[lo:hi] = clique[0:lo] & ((adj[b] & rest) == rest)
    maximal = clique.copy()
    maximal[0] = False
    for v in range(n):
        outside = (S >> v) & 1 == 0
        extends = (adj[v] & S) == S
        maximal &= ~(outside & extends)
    out = []
    for s in np.nonzero(maximal)[0]:
        s = int(s)
        out.append(tuple(i for i in range(n) if (s >> i) & 1))
    return out


def core_numbers_by_definition(n, row_ptr, col_idx):
    """core(v) = largest k such that v lies in a subgraph of minimum degree >= k,
    found for each k by deleting vertices of degree < k until none remain."""
    adj = [set(int(x) for x in col_idx[row_ptr[v]:row_ptr[v + 1]]) for v in range(n)]
    core = [0] * n
    k = 1
    while True:
        alive = set(range(n))
        changed = True
        while changed:
            changed = False
            for v in list(alive):
                if len(adj[v] & alive) < k:
                    alive.discard(v)
                    changed = True
        if not alive:
            return core
        for v in alive:
            core[v] = k
        k += 1
