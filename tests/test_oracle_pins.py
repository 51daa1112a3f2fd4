"""Pins for the oracle, against facts that do not come from the oracle itself:
brute-force subset enumeration, closed-form graph families, the worked example of
section 2.1 ("Parallelizing Maximal Clique Enumeration on GPUs"), the textbook
definition of core numbers, and clique/maximality invariants."""
import itertools

import numpy as np
import pytest

import mce_inputs as mi
import oracle
from tests import brute
from tests.golden.load import read_fixture


def summary_of(g):
    r = oracle.mce(g.n, g.row_ptr, g.col_idx)
    assert r.complete
    return r.count, r.hash, r.hist


def expect(cliques):
    c, h, hist = brute.set_summary(cliques)
    return c, h, hist


# ------------------------------------------------------------------ the mixer
def test_mix64_matches_python_ints():
    rng = np.random.default_rng(7)
    vals = [0, 1, 2 ** 63, 2 ** 64 - 1] + [int(x) for x in rng.integers(0, 2 ** 63, 200)]
    for v in vals:
        assert oracle.mix64(v) == brute.mix64(v)


def test_clique_hash_is_a_set_function_and_spreads():
    rng = np.random.default_rng(8)
    seen = set()
    for _ in range(3000):
        k = int(rng.integers(1, 12))
        c = rng.choice(10 ** 6, size=k, replace=False)
        h = oracle.clique_hash(c)
        assert h == brute.clique_hash(c.tolist())
        assert h == oracle.clique_hash(rng.permutation(c))     # order-free
        seen.add(h)
    assert len(seen) == 3000                                   # no collisions


# ------------------------------------------------------------------ worked example
def test_fig1a_two_maximal_cliques():
    fx = read_fixture("fig1a.txt")
    g = mi.fig1a()
    assert sorted(map(tuple, g.edge_list().tolist())) == sorted(fx["edges"])
    assert int(g.degrees()[0]) == fx["degree"][0] == fx["maxdegree"]
    cl = oracle.list_cliques(g.n, g.row_ptr, g.col_idx)
    assert sorted(cl) == sorted(fx["maximal"])
    for nm in fx["not_maximal"]:
        assert nm not in cl
    assert summary_of(g) == expect(fx["maximal"])
    assert summary_of(g)[2] == [0, 0, 0, 1, 1]


# ------------------------------------------------------------------ brute force
@pytest.mark.parametrize("seed", range(60))
def test_oracle_equals_brute_force_small(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 13))
    p = float(rng.choice([0.0, 0.1, 0.3, 0.5, 0.7, 0.9, 1.0]))
    g = mi.random_small(n, p, seed)
    want = brute.brute_maximal_cliques(g.n, g.row_ptr, g.col_idx)
    assert summary_of(g) == expect(want)
    assert sorted(oracle.list_cliques(g.n, g.row_ptr, g.col_idx)) == sorted(want)


@pytest.mark.parametrize("seed,n,p", [(100, 16, 0.5), (101, 18, 0.6), (102, 18, 0.8),
                                      (103, 20, 0.7), (104, 20, 0.85), (105, 17, 0.95)])
def test_oracle_equals_brute_force_larger(seed, n, p):
    g = mi.random_small(n, p, seed)
    want = brute.brute_maximal_cliques(g.n, g.row_ptr, g.col_idx)
    assert summary_of(g) == expect(want)


# ------------------------------------------------------------------ closed forms
@pytest.mark.parametrize("n", [1, 2, 3, 5, 17, 64, 65, 130])
def test_complete_graph_has_one_clique(n):
    assert summary_of(mi.complete(n)) == expect([tuple(range(n))])


@pytest.mark.parametrize("n", [0, 1, 7, 100])
def test_empty_graph_has_n_singletons(n):
    assert summary_of(mi.empty(n)) == expect([(i,) for i in range(n)])


@pytest.mark.parametrize("n", [4, 5, 9, 200])
def test_cycle_has_n_edges_as_cliques(n):
    want = [tuple(sorted((i, (i + 1) % n))) for i in range(n)]
    assert summary_of(mi.cycle(n)) == expect(want)


def test_star_path_petersen_are_their_edges():
    for g in (mi.star(9), mi.path(12), mi.petersen()):
        el = [tuple(e) for e in g.edge_list().tolist()]   # triangle-free, no isolated vertices
        assert summary_of(g) == expect(el)


def _product_summary(parts):
    """(count, hash, hist) of the complete multipartite graph with these vertex
    groups, computed by listing one vertex per group (numpy uint64 arithmetic)."""
    with np.errstate(over="ignore"):
        g = np.uint64(brute.GOLDEN)

        def mix(z):
            z = z ^ (z >> np.uint64(30))
            z = z * np.uint64(0xBF58476D1CE4E5B9)
            z = z ^ (z >> np.uint64(27))
            z = z * np.uint64(0x94D049BB133111EB)
            return z ^ (z >> np.uint64(31))

        sums = np.zeros(1, np.uint64)
        for grp in parts:
            h = mix(np.asarray(grp, np.uint64) + g)
            sums = (sums[:, None] + h[None, :]).ravel()
        k = len(parts)
        total = mix(sums + np.uint64(k) * g).sum(dtype=np.uint64)
    hist = [0] * (k + 1)
    hist[k] = int(sums.size)
    return int(sums.size), int(total), hist


@pytest.mark.parametrize("k", [1, 2, 4, 7, 10])
def test_moon_moser_has_3_to_the_k(k):
    g = mi.moon_moser(3 * k)
    got = summary_of(g)
    assert got[0] == 3 ** k
    assert got == _product_summary([[3 * t, 3 * t + 1, 3 * t + 2] for t in range(k)])


def test_moon_moser_45_closed_form():
    g = mi.moon_moser(45)
    assert g.m == 945
    got = summary_of(g)
    assert got[0] == 14_348_907 == 3 ** 15
    assert got == _product_summary([[3 * t, 3 * t + 1, 3 * t + 2] for t in range(15)])


@pytest.mark.parametrize("sizes", [[1, 2, 3], [4, 4], [2, 5, 1, 3], [6, 1, 1, 1, 2]])
def test_complete_multipartite_is_a_product(sizes):
    g = mi.complete_multipartite(sizes)
    parts, off = [], 0
    for s in sizes:
        parts.append(list(range(off, off + s)))
        off += s
    assert summary_of(g) == _product_summary(parts)


# ------------------------------------------------------------------ invariants
@pytest.mark.parametrize("seed", range(8))
def test_listed_cliques_are_maximal_and_distinct(seed):
    g = mi.random_small(40, 0.3 + 0.08 * seed, 1000 + seed)
    adj = [set(g.col_idx[g.row_ptr[v]:g.row_ptr[v + 1]].tolist()) for v in range(g.n)]
    cl = oracle.list_cliques(g.n, g.row_ptr, g.col_idx)
    assert len(set(cl)) == len(cl)
    covered = set()
    for c in cl:
        for a, b in itertools.combinations(c, 2):
            assert b in adj[a]                              # a clique
            covered.add((a, b))
        common = set(range(g.n)) if not c else set.intersection(*(adj[x] for x in c))
        assert not (common - set(c))                        # maximal
    for v in range(g.n):                                    # every edge is covered
        for u in adj[v]:
            if v < u:
                assert (v, u) in covered
    # the bitset search and the list search agree
    assert summary_of(g) == expect(cl)


@pytest.mark.parametrize("seed", range(6))
def test_relabelling_and_disjoint_union(seed):
    rng = np.random.default_rng(seed)
    g = mi.random_small(30, 0.5, 2000 + seed)
    perm = rng.permutation(g.n)
    cl = oracle.list_cliques(g.n, g.row_ptr, g.col_idx)
    moved = [tuple(sorted(int(perm[x]) for x in c)) for c in cl]
    gr = mi.relabel(g, perm)
    assert summary_of(gr) == expect(moved)
    h = mi.random_small(25, 0.6, 3000 + seed)
    u = mi.disjoint_union(g, h)
    a, b = summary_of(g), summary_of(h)
    c = summary_of(u)
    assert c[0] == a[0] + b[0]
    hist = [0] * max(len(a[2]), len(b[2]))
    for i, x in enumerate(a[2]):
        hist[i] += x
    for i, x in enumerate(b[2]):
        hist[i] += x
    assert c[2] == hist
    shifted = [tuple(x + g.n for x in cc) for cc in oracle.list_cliques(h.n, h.row_ptr, h.col_idx)]
    assert c == expect(cl + shifted)


# ------------------------------------------------------------------ ordering
@pytest.mark.parametrize("seed", range(25))
def test_peel_core_numbers_match_definition(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    g = mi.random_small(n, float(rng.uniform(0.05, 0.9)), 4000 + seed)
    core, rnd, d = oracle.peel(g.n, g.row_ptr, g.col_idx)
    assert core.tolist() == brute.core_numbers_by_definition(g.n, g.row_ptr, g.col_idx)
    assert d == (max(core) if n else 0)
    # degeneracy order: each vertex has at most d later neighbours
    for v in range(g.n):
        later = [u for u in g.col_idx[g.row_ptr[v]:g.row_ptr[v + 1]]
                 if (rnd[u], u) > (rnd[v], v)]
        assert len(later) <= core[v] <= d


def test_peel_known_families():
    for g, d in [(mi.complete(9), 8), (mi.cycle(11), 2), (mi.path(7), 1), (mi.star(6), 1),
                 (mi.moon_moser(45), 42), (mi.empty(5), 0), (mi.petersen(), 3)]:
        core, rnd, dd = oracle.peel(g.n, g.row_ptr, g.col_idx)
        assert dd == d, g.name
    # a regular graph is peeled in a single round
    core, rnd, d = oracle.peel(*(lambda g: (g.n, g.row_ptr, g.col_idx))(mi.moon_moser(45)))
    assert set(rnd.tolist()) == {0} and set(core.tolist()) == {42}
    # a path loses its two ends first: rounds grow toward the middle
    core, rnd, d = oracle.peel(*(lambda g: (g.n, g.row_ptr, g.col_idx))(mi.path(7)))
    assert rnd.tolist() == [0, 1, 2, 3, 2, 1, 0]


def test_roots_partition_adds_up():
    g = mi.random_small(60, 0.35, 77)
    whole = oracle.mce(g.n, g.row_ptr, g.col_idx)
    _, rnd, _ = oracle.peel(g.n, g.row_ptr, g.col_idx)
    cl = oracle.list_cliques(g.n, g.row_ptr, g.col_idx)
    parts = [list(range(0, 20)), list(range(20, 41)), list(range(41, 60))]
    tot_c, tot_h, tot_hist = 0, 0, [0] * len(whole.hist)
    for part in parts:
        r = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=np.array(part, np.int32))
        # the cliques of a root set are those whose earliest vertex is in it
        mine = [c for c in cl if min(c, key=lambda x: (rnd[x], x)) in set(part)]
        assert (r.count, r.hash, r.hist) == expect(mine) or (r.count == 0 and not mine)
        tot_c += r.count
        tot_h = (tot_h + r.hash) & brute.M64
        for i, x in enumerate(r.hist):
            tot_hist[i] += x
    assert (tot_c, tot_h, tot_hist) == (whole.count, whole.hash, whole.hist)


# ------------------------------------------------------------------ second-level subtrees
def summary_l2(g, roots=None):
    r = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=roots, level=2)
    assert r.complete
    return r.count, r.hash, r.hist


@pytest.mark.parametrize("seed", range(40))
def test_second_level_equals_brute_force(seed):
    """Algorithm 4 (one subtree per edge {r, w}, w after r, plus isolated
    vertices) finds exactly the maximal cliques that subset enumeration finds."""
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(0, 16))
    p = float(rng.choice([0.0, 0.1, 0.3, 0.5, 0.7, 0.9, 1.0]))
    g = mi.random_small(n, p, 1000 + seed)
    assert summary_l2(g) == expect(brute.brute_maximal_cliques(g.n, g.row_ptr, g.col_idx))


def test_second_level_closed_forms():
    assert summary_l2(mi.complete(40)) == expect([tuple(range(40))])
    assert summary_l2(mi.empty(9)) == expect([(i,) for i in range(9)])
    assert summary_l2(mi.cycle(11)) == expect([tuple(sorted((i, (i + 1) % 11))) for i in range(11)])
    g = mi.moon_moser(24)
    assert summary_l2(g) == _product_summary([[3 * t, 3 * t + 1, 3 * t + 2] for t in range(8)])
    g = mi.disjoint_union(mi.complete(5), mi.empty(3), mi.star(4))
    assert summary_l2(g) == summary_of(g)


def test_second_level_root_sets_are_first_level_root_sets():
    """Per root set, both decompositions give the cliques whose earliest vertex
    is in the set: L2 subtrees of edges leaving a root carry exactly those."""
    g = mi.chung_lu(3000, 8.0, 2.3, None, 5, planted=6, planted_min=8, planted_max=14)
    rng = np.random.default_rng(3)
    roots = np.sort(rng.choice(g.n, size=400, replace=False)).astype(np.int32)
    a = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=roots)
    b = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=roots, level=2)
    assert a.key() == b.key()
    assert summary_l2(g) == summary_of(g)


def test_node_budget_stops():
    g = mi.moon_moser(30)
    r = oracle.mce(g.n, g.row_ptr, g.col_idx, node_budget=1000)
    assert not r.complete and r.nodes == 1001


# ------------------------------------------------------------------ validation
def test_validate_classes():
    g = mi.random_small(12, 0.5, 5)
    assert oracle.validate(g.n, g.row_ptr, g.col_idx) == 0
    rp, ci = g.row_ptr.copy(), g.col_idx.copy()
    bad = ci.copy(); bad[0] = g.n
    assert oracle.validate(g.n, rp, bad) & oracle.OV_RANGE
    # self loop on vertex 0 (keep the row sorted)
    v = 0
    row = ci[rp[v]:rp[v + 1]].copy()
    bad = ci.copy(); bad[rp[v]] = v
    assert oracle.validate(g.n, rp, bad) & (oracle.OV_LOOP | oracle.OV_ASYM)
    bad = ci.copy()
    r0 = int(np.argmax(np.diff(rp) >= 2))
    bad[rp[r0]], bad[rp[r0] + 1] = bad[rp[r0] + 1], bad[rp[r0]]
    assert oracle.validate(g.n, rp, bad) & oracle.OV_ORDER
    badrp = rp.copy(); badrp[-1] += 1
    assert oracle.validate(g.n, badrp, ci) & oracle.OV_ROWPTR
    # drop one direction of an edge
    u, w = map(int, g.edge_list()[0])
    keep = np.ones(ci.size, bool)
    keep[rp[u] + int(np.nonzero(ci[rp[u]:rp[u + 1]] == w)[0][0])] = False
    rp2 = rp.copy(); rp2[u + 1:] -= 1
    assert oracle.validate(g.n, rp2, ci[keep]) == oracle.OV_ASYM
    del row


# ---------------------------------------------------------------- subtree size estimate
# Knuth's random probe (oracle.knuth) sizes the workloads before they are
# enumerated. On graphs whose pivoted search tree is regular every walk is
# exact; elsewhere the estimator is unbiased, so its mean over many walks must
# sit within a few standard errors of the exact enumeration (the oracle,
# pinned above by brute force and closed forms).
@pytest.mark.parametrize("g", [mi.moon_moser(15), mi.moon_moser(18), mi.complete_multipartite([3, 3, 3, 3]),
                               mi.complete_multipartite([2, 2, 2, 2, 2]), mi.complete(9)])
def test_knuth_exact_on_regular_trees(g):
    _, rnd, _ = oracle.peel(g.n, g.row_ptr, g.col_idx)
    total = 0.0
    for r in range(g.n):
        e = oracle.knuth(g.n, g.row_ptr, g.col_idx, r, 40, seed=r + 1, rnd=rnd)
        ex = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=[r], rnd=rnd)
        assert e.cliques_se == 0 and e.nodes_se == 0      # every walk gives the same product
        assert e.cliques == ex.count and e.nodes == ex.nodes
        total += e.cliques
    # closed forms: 3^(n/3) for Moon-Moser, the product of part sizes for a complete multipartite graph
    assert total == oracle.mce(g.n, g.row_ptr, g.col_idx).count


def test_knuth_moon_moser_closed_form():
    g = mi.moon_moser(45)
    e = oracle.knuth(g.n, g.row_ptr, g.col_idx, 0, 8, seed=5)
    assert e.cliques == 3 ** 14 and e.cliques_se == 0      # the cliques through vertex 0
    assert e.max_depth == 14                               # one walk ends at a 15-vertex clique


@pytest.mark.parametrize("seed", range(4))
def test_knuth_unbiased_against_enumeration(seed):
    worst, spread = 0.0, 0
    for n, p in ((40, 0.5), (60, 0.3), (30, 0.7)):
        g = mi.random_small(n, p, seed)
        _, rnd, _ = oracle.peel(g.n, g.row_ptr, g.col_idx)
        for r in range(0, n, 7):
            e = oracle.knuth(g.n, g.row_ptr, g.col_idx, r, 4000, seed=11 + r, rnd=rnd)
            ex = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=[r], rnd=rnd)
            for est, se, exact in ((e.cliques, e.cliques_se, ex.count), (e.nodes, e.nodes_se, ex.nodes)):
                if se == 0:
                    assert est == exact
                else:
                    spread += 1
                    worst = max(worst, abs(est - exact) / se)
    assert spread > 10          # the walks did vary: the test compares means, not single paths
    assert worst < 6.0


@pytest.mark.parametrize("seed,n,p", [(200, 14, 0.5), (201, 18, 0.7), (202, 20, 0.85), (203, 16, 0.3)])
def test_per_root_runs_add_up_to_brute_force(seed, n, p):
    """oracle.mce_each (one node budget per subtree) over every root gives the
    brute-force clique count and hash; a budget below a subtree's size leaves
    that root unfinished."""
    g = mi.random_small(n, p, seed)
    _, rnd, _ = oracle.peel(g.n, g.row_ptr, g.col_idx)
    roots = np.arange(g.n, dtype=np.int32)
    nodes, cnt, hsh, done = oracle.mce_each(g.n, g.row_ptr, g.col_idx, roots, 0, rnd)
    want = brute.brute_maximal_cliques(g.n, g.row_ptr, g.col_idx)
    wc, wh, _ = brute.set_summary(want)
    assert done.all()
    assert int(cnt.sum()) == wc
    assert int(hsh.sum(dtype=np.uint64)) == wh
    big = int(np.argmax(nodes))
    if nodes[big] > 1:
        _, _, _, d2 = oracle.mce_each(g.n, g.row_ptr, g.col_idx, roots[big:big + 1], int(nodes[big]) - 1, rnd)
        assert d2[0] == 0
        _, c3, _, d3 = oracle.mce_each(g.n, g.row_ptr, g.col_idx, roots[big:big + 1], int(nodes[big]), rnd)
        assert d3[0] == 1 and c3[0] == cnt[big]


# ------------------------------------------------------------------ a root's bit-encoded subgraph
def _dense_table(g, rnd, root, W, micro, full):
    """The same words from a dense adjacency matrix and Python integers."""
    n = g.n
    A = np.zeros((n, n), bool)
    src = np.repeat(np.arange(n), np.diff(g.row_ptr))
    A[src, g.col_idx] = True
    nb = sorted(int(u) for u in np.nonzero(A[root])[0])
    lat = lambda u: (int(rnd[u]), u) > (int(rnd[root]), root)
    P = [u for u in nb if lat(u)]
    X = [u for u in nb if not lat(u)]
    G = 0x9E3779B97F4A7C15
    words = [len(P) | (len(X) << 32), root | (1 << 32), brute.mix64(root + G)]
    for m in P + (X if full else []):
        row = sum(1 << b for b, u in enumerate(P) if A[m, u])
        words += [(row >> (64 * i)) & (2 ** 64 - 1) for i in range(W)]
    if micro:
        words += [sum(1 << a for a, u in enumerate(X) if A[v, u]) for v in P]
    words += [brute.mix64(u + G) for u in P]
    ids = P + X
    words += [ids[j] | ((ids[j + 1] if j + 1 < len(ids) else 0) << 32) for j in range(0, len(ids), 2)]
    return np.array(words, dtype=np.uint64)


@pytest.mark.parametrize("seed", range(6))
def test_root_table_matches_dense_adjacency(seed):
    g = mi.random_small(70, 0.35 if seed % 2 else 0.15, seed)
    _, rnd, _ = oracle.peel(g.n, g.row_ptr, g.col_idx)
    for root in range(g.n):
        for W, micro, full in [(1, True, True), (1, False, True), (1, False, False), (2, False, True)]:
            deg = int(g.row_ptr[root + 1] - g.row_ptr[root])
            got = oracle.root_table(g.n, g.row_ptr, g.col_idx, rnd, root, W, micro, full)
            want = _dense_table(g, rnd, root, W, micro, full)
            assert np.array_equal(got, want), (seed, root, W, micro, full, deg)
