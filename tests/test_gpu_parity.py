"""GPU parity: the HIP engine, called through the C ABI, against the oracle.

Every case compares count, histogram and hash element by element (integer work:
the bar is bit-exact). Inputs are seeded synthetic graphs from mce_inputs.
"""
import numpy as np
import pytest

import mce_inputs as mi
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # pragma: no cover - CPU-only runs deselect these
    pytest.skip("needs a GPU", allow_module_level=True)

import maximal_clique_enumeration_amd as mce  # noqa: E402

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module", params=["partial", "full", "partial-nomicro", "full-nomicro", "partial-l2",
                                        "full-l2"])
def eng(request):
    """One engine per induced-subgraph encoding (section 3.4), with the micro
    kernel (one search-tree node per lane for subtrees with |P|, |X| <= 64) on
    and off, and with second-level subtrees (section 3.2): every case that takes
    this fixture runs under all six."""
    if not mce.lib_built():
        from maximal_clique_enumeration_amd import build
        build.build()
    sub, _, opt = request.param.partition("-")
    e = mce.Engine(device=0, timeout_ms=20000, subgraph=sub, micro=opt != "nomicro", level=2 if opt == "l2" else 1)
    yield e
    e.close()


def on_gpu(g):
    return torch.from_numpy(g.row_ptr).to(DEV), torch.from_numpy(g.col_idx).to(DEV)


def check(eng, g, roots=None):
    rp, ci = on_gpu(g)
    r = None if roots is None else torch.from_numpy(np.asarray(roots, np.int32)).to(DEV)
    print(f"case {g.name} n={g.n} m={g.m}", flush=True)
    got = eng.run(rp, ci, roots=r)
    want = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=roots)
    assert want.complete
    assert got.count == want.count, (g.name, got, want)
    assert got.hist == want.hist, (g.name, got.hist, want.hist)
    assert got.hash == want.hash, (g.name, hex(got.hash), hex(want.hash))
    return got


# ------------------------------------------------------------------ small worked cases
def test_fig1a(eng):
    got = check(eng, mi.fig1a())
    assert got.count == 2 and got.hist == [0, 0, 0, 1, 1]


@pytest.mark.parametrize("n", [1, 2, 3, 17, 64, 65, 66, 129, 130, 200])
def test_complete(eng, n):
    got = check(eng, mi.complete(n))
    assert got.count == 1 and len(got.hist) == n + 1


@pytest.mark.parametrize("n", [1, 5, 1000])
def test_empty(eng, n):
    got = check(eng, mi.empty(n))
    assert got.count == n


@pytest.mark.parametrize("n", [4, 7, 100, 5000])
def test_cycle(eng, n):
    got = check(eng, mi.cycle(n))
    assert got.count == n


@pytest.mark.parametrize("k", [1, 2, 5, 9, 12])
def test_moon_moser(eng, k):
    got = check(eng, mi.moon_moser(3 * k))
    assert got.count == 3 ** k


def test_moon_moser_45_full(eng):
    """The bench workload, whole graph: 3^15 maximal cliques of size 15."""
    got = check(eng, mi.config_graph(1))
    assert got.count == 14_348_907 and got.hist[15] == 14_348_907


@pytest.mark.parametrize("seed", range(40))
def test_random_small(eng, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 90))
    p = float(rng.choice([0.05, 0.2, 0.4, 0.6, 0.8, 0.95]))
    check(eng, mi.random_small(n, p, 500 + seed))


@pytest.mark.parametrize("n,p,seed", [(300, 0.3, 1), (200, 0.5, 2), (160, 0.7, 3), (400, 0.4, 4),
                                      (300, 0.5, 4)])
def test_random_dense(eng, n, p, seed):
    """Roots with |P| above 64 and 128 (bitset widths 2 and 4 words), deep trees."""
    check(eng, mi.random_small(n, p, seed))


@pytest.mark.parametrize("sizes", [[2, 3, 4, 5], [1] * 70, [3, 1, 4, 1, 5, 9, 2, 6],
                                   [3] * 5 + [1] * 300, [2] * 10 + [1] * 600, [2] * 3 + [1] * 1200])
def test_multipartite(eng, sizes):
    """Complete multipartite graphs: prod(sizes) cliques of size len(sizes); the
    large ones put |P| near 300, 600 and 1200 (widths 8, 16 and 32 words)."""
    got = check(eng, mi.complete_multipartite(sizes))
    assert got.count == int(np.prod(sizes))


def test_more_hubs_than_bitmaps():
    """Second-level runs give vertices of degree >= 256 an adjacency bitmap, at
    most 1024 of them. K_{600,600} has 1200 such vertices, so some rows are
    tested with bitmaps and the others with binary searches; every edge is a
    maximal clique (the common neighbourhoods are empty)."""
    g = mi.complete_multipartite([600, 600])
    with mce.Engine(device=0, timeout_ms=20000, level=2) as e:
        got = check(e, g)
        assert got.count == 600 * 600 and got.hist == [0, 0, 600 * 600]


@pytest.mark.parametrize("core", [300, 700, 1100])
def test_hub_rows(eng, core):
    """Core roots of widths 8, 16 and 32 words whose X holds hubs: the hub rows
    (degree far above 2 |P|) are built by probing P members in the CSR row, the
    core rows by streaming, each root's slabs over many blocks."""
    check(eng, mi.hub_clique(core, 4, 3000, 0.7, 12, core))


def test_er_2000(eng):
    """The small configuration: G(2000, 0.01), seed 1."""
    check(eng, mi.config_graph(0))


def test_chung_lu_with_planted_cliques(eng):
    """A power-law graph with overlapping planted cliques: long X_X arrays."""
    check(eng, mi.chung_lu(20000, 12.0, 2.3, None, 3, planted=40, planted_min=10, planted_max=30))


def test_disjoint_union_and_isolated(eng):
    g = mi.disjoint_union(mi.moon_moser(15), mi.empty(7), mi.cycle(9), mi.complete(70))
    check(eng, g)


# ------------------------------------------------------------------ ordering
@pytest.mark.parametrize("make", [lambda: mi.config_graph(0), lambda: mi.moon_moser(45),
                                  lambda: mi.chung_lu(30000, 15.0, 2.2, None, 9, planted=10),
                                  lambda: mi.chung_lu(200000, 20.0, 2.3, None, 11, planted=50),
                                  lambda: mi.path(40), lambda: mi.random_small(500, 0.3, 4),
                                  # grid peels that hand the residual graph to block 0 at once: one
                                  # round of 30,000 vertices, 20,000 rounds of two, a 10,000-entry
                                  # row compacted in spans
                                  lambda: mi.cycle(30000), lambda: mi.path(40000),
                                  lambda: mi.chung_lu(40000, 20.0, 2.1, 8000.0, 5),
                                  lambda: mi.disjoint_union(mi.complete_multipartite([1, 10000]), mi.cycle(20000),
                                                            mi.chung_lu(20000, 12.0, 2.0, 9000.0, 7)),
                                  # a hub of degree 40,000 keeps the grid until it is gone
                                  lambda: mi.complete_multipartite([1, 40000])])
def test_ordering_matches_oracle(eng, make):
    g = make()
    rp, ci = on_gpu(g)
    eng.run(rp, ci)
    core, rnd = eng.ordering(g.n)
    ocore, ornd, d = oracle.peel(g.n, g.row_ptr, g.col_idx)
    assert np.array_equal(core.cpu().numpy(), ocore)
    assert np.array_equal(rnd.cpu().numpy(), ornd)
    info = eng.graph_info()
    assert info["degeneracy"] == d and info["rounds"] == int(ornd.max()) + 1
    assert info["max_degree"] == int(g.degrees().max())


# ------------------------------------------------------------------ split peel
def test_split_peel_handover_order():
    """More vertices than the peel's tail takes: the grid hands the tail to a
    one-block launch, and the whole search runs beside it in the hand-over
    order (the vertices gone before the tail by round, then the tail's by their
    degree among themselves, then id). The cliques match the oracle and a serial
    run (the peel's order), and the peel's order itself matches the oracle's,
    run after run."""
    g = mi.chung_lu(200000, 20.0, 2.3, None, 11, planted=50)
    rp, ci = on_gpu(g)
    print(f"case {g.name} n={g.n} m={g.m}, split peel", flush=True)
    want = oracle.mce(g.n, g.row_ptr, g.col_idx)
    ocore, ornd, d = oracle.peel(g.n, g.row_ptr, g.col_idx)
    with mce.Engine(device=0, timeout_ms=60000) as eo, \
            mce.Engine(device=0, timeout_ms=60000, overlap=False) as es:
        for _ in range(2):
            for e in (eo, es):
                got = e.run(rp, ci)
                assert (got.count, got.hist, got.hash) == (want.count, want.hist, want.hash)
                core, rnd = e.ordering(g.n)
                assert np.array_equal(core.cpu().numpy(), ocore) and np.array_equal(rnd.cpu().numpy(), ornd)
                info = e.graph_info()
                assert info["roots_started"] == g.n and info["degeneracy"] == d
                assert info["rounds"] == int(ornd.max()) + 1
        so, ss = eo.stats(), es.stats()
        r0 = so["handover_round"]
        assert ss["handover_round"] == -1 and 0 < r0 <= int(ornd.max())
        # the vertices still present at the hand-over: at most the tail's capacity
        assert 0 < int((ornd >= r0).sum()) <= 65535


# ------------------------------------------------------------------ root subsets
def test_root_subsets(eng):
    g = mi.chung_lu(20000, 12.0, 2.3, None, 5, planted=20, planted_min=8, planted_max=25)
    rng = np.random.default_rng(3)
    roots = rng.choice(g.n, size=3000, replace=False).astype(np.int32)
    check(eng, g, roots=roots)
    check(eng, g, roots=roots[:1])
    check(eng, g, roots=np.zeros(0, np.int32))


# ------------------------------------------------------------------ stress matrix
@pytest.mark.parametrize("micro", [True, False])
@pytest.mark.parametrize("worker_list", [False, True])
@pytest.mark.parametrize("donate_min_p", [1, 10, 1 << 20])
@pytest.mark.parametrize("max_workers", [1, 2, 7, 0])
def test_stress_matrix(worker_list, donate_min_p, max_workers, micro):
    graphs = [mi.moon_moser(30), mi.random_small(120, 0.5, 8),
              mi.chung_lu(5000, 10.0, 2.3, None, 2, planted=10, planted_min=8, planted_max=20)]
    donations = 0
    with mce.Engine(device=0, worker_list=worker_list, donate_min_p=donate_min_p,
                    micro_donate_min_p=donate_min_p, max_workers=max_workers, timeout_ms=20000,
                    micro=micro) as e:
        for g in graphs:
            check(e, g)
            donations += e.stats()["donations"]
    if not worker_list or donate_min_p == 1 << 20 or max_workers == 1:
        assert donations == 0


@pytest.mark.parametrize("micro", [True, False])
@pytest.mark.parametrize("max_workers", [2, 7, 64, 0])
def test_single_root_is_shared(max_workers, micro):
    """One first-level subtree (root 0 of the Moon-Moser graph on 45 vertices,
    3^14 maximal cliques) and idle wavefronts: the worker list must hand branches
    over, and the result must not change."""
    g = mi.moon_moser(45)
    with mce.Engine(device=0, donate_min_p=1, max_workers=max_workers, timeout_ms=20000, micro=micro) as e:
        got = check(e, g, roots=np.array([0], np.int32))
        assert got.count == 3 ** 14
        st = e.stats()
        assert st["donations"] > 0 and st["leaves"] == 3 ** 14
        assert st["micro_roots"] == (1 if micro else 0)


def test_micro_routing():
    """Subtrees with |P| <= 64 and |X| <= 64 go to the micro kernel unless it is
    switched off; larger ones never do. The frame stack stays far below its
    4096-frame capacity (an overflow is reported as MCE_ERR_LIMIT)."""
    g = mi.chung_lu(20000, 12.0, 2.3, None, 5, planted=20, planted_min=8, planted_max=25)
    deg = g.degrees()
    with mce.Engine(device=0, timeout_ms=20000) as e:
        check(e, g)
        st = e.stats()
        info = e.graph_info()
        assert 0 < st["micro_roots"] <= int((deg > 0).sum())
        assert info["max_x"] > 64 and st["launches"] >= 2   # the hubs go to the wavefront kernels
        assert 0 < st["max_stack_frames"] < 4096
    with mce.Engine(device=0, timeout_ms=20000, micro=False) as e:
        check(e, g)
        assert e.stats()["micro_roots"] == 0 and e.stats()["max_stack_frames"] == 0


def test_hbm_staging_and_repeats():
    g = mi.moon_moser(36)
    want = oracle.mce(g.n, g.row_ptr, g.col_idx)
    rp, ci = on_gpu(g)
    for hbm in (False, True):
        with mce.Engine(device=0, hbm_staging=hbm, timeout_ms=20000) as e:
            for _ in range(5):
                assert e.run(rp, ci).key() == want.key()


# ------------------------------------------------------------------ input checks
def _bad(eng, n, rp, ci):
    trp = torch.from_numpy(np.asarray(rp, np.int32)).to(DEV)
    tci = torch.from_numpy(np.asarray(ci, np.int32)).to(DEV)
    with pytest.raises(mce.MceError) as ex:
        eng.run(trp, tci)
    assert ex.value.status == mce.MCE_ERR_GRAPH
    return eng.graph_info()["graph_errors"]


@pytest.mark.parametrize("make", [lambda: mi.random_small(12, 0.5, 5), lambda: mi.erdos_renyi(6000, 0.002, 3)])
def test_rejects_malformed(eng, make):
    """Each kind of malformed CSR is rejected: on a small graph (checked by one
    block) and on a larger one (the grid checks: rows in 16-lane groups)."""
    g = make()
    rp, ci = g.row_ptr.copy(), g.col_idx.copy()
    bad = ci.copy(); bad[0] = g.n
    assert _bad(eng, g.n, rp, bad) & mce.MCE_GRAPH_RANGE
    bad = ci.copy(); bad[rp[0]] = 0
    assert _bad(eng, g.n, rp, bad) & (mce.MCE_GRAPH_LOOP | mce.MCE_GRAPH_ASYM)
    r0 = int(np.argmax(np.diff(rp) >= 2))
    bad = ci.copy(); bad[rp[r0]], bad[rp[r0] + 1] = bad[rp[r0] + 1], bad[rp[r0]]
    assert _bad(eng, g.n, rp, bad) & mce.MCE_GRAPH_ORDER
    badrp = rp.copy(); badrp[3] = badrp[4] + 1
    assert _bad(eng, g.n, badrp, ci) & mce.MCE_GRAPH_ROWPTR
    u, w = map(int, g.edge_list()[0])
    keep = np.ones(ci.size, bool)
    keep[rp[u] + int(np.nonzero(ci[rp[u]:rp[u + 1]] == w)[0][0])] = False
    rp2 = rp.copy(); rp2[u + 1:] -= 1
    assert _bad(eng, g.n, rp2, ci[keep]) == mce.MCE_GRAPH_ASYM
    # the engine still works afterwards
    check(eng, g)


def _drop_edge(rp, ci, u, w):
    """The CSR without the directed edge (u, w)."""
    pos = rp[u] + int(np.nonzero(ci[rp[u]:rp[u + 1]] == w)[0][0])
    keep = np.ones(ci.size, bool)
    keep[pos] = False
    rp2 = rp.copy()
    rp2[u + 1:] -= 1
    return rp2, ci[keep]


def test_asymmetry_on_either_side(eng):
    """Symmetry is searched only for edges stored at the endpoint later in
    (degree, id) order, and completed by counting: a missing reverse must be
    found whichever endpoint stores the surviving edge, also in a hub row of
    thousands of edges (whose entries several wavefronts share)."""
    g = mi.hub_clique(300, 4, 3000, 0.7, 12, 7)
    rp, ci = g.row_ptr, g.col_idx
    deg = np.diff(rp)
    hub = int(np.argmax(deg))
    assert deg[hub] > 2048
    leaf = int(ci[rp[hub]])                    # a neighbour of the hub of smaller degree
    core = int(ci[rp[hub + 1] - 1]) if deg[int(ci[rp[hub + 1] - 1])] > 1 else leaf
    a, b = map(int, g.edge_list()[len(g.edge_list()) // 2])
    for u, w in [(hub, leaf), (leaf, hub), (hub, core), (core, hub), (a, b), (b, a)]:
        rp2, ci2 = _drop_edge(rp, ci, u, w)
        assert _bad(eng, g.n, rp2, ci2) == mce.MCE_GRAPH_ASYM, (u, w)
    check(eng, g)


@pytest.mark.parametrize("n, m, seed", [(100000, 400, 1), (70001, 2500, 2)])
def test_long_runs_of_empty_rows(eng, n, m, seed):
    """Entries are checked in 64-entry tiles whose rows are found among the next
    64 row ends; between two edges lie hundreds of empty rows here, so a tile's
    rows are found over many such loads. The graph's cliques match the oracle
    (every isolated vertex is a maximal clique of one), and a missing reverse
    edge anywhere is still found."""
    rng = np.random.default_rng(seed)
    u = rng.integers(0, n, m)
    v = rng.integers(0, n, m)
    g = mi.from_edges(n, u, v, f"sparse{n}")
    check(eng, g)
    rp, ci = g.row_ptr, g.col_idx
    pairs = g.edge_list()
    for k in (0, len(pairs) // 2, len(pairs) - 1):
        x, y = map(int, pairs[k])
        for s, t in ((x, y), (y, x)):
            rp2, ci2 = _drop_edge(rp, ci, s, t)
            assert _bad(eng, g.n, rp2, ci2) == mce.MCE_GRAPH_ASYM, (s, t)


def test_bad_roots_and_empty_graph(eng):
    g = mi.cycle(10)
    rp, ci = on_gpu(g)
    with pytest.raises(mce.MceError) as ex:
        eng.run(rp, ci, roots=torch.tensor([3, 10], dtype=torch.int32, device=DEV))
    assert ex.value.status == mce.MCE_ERR_ARG
    e0 = mi.empty(0)
    got = eng.run(*on_gpu(e0))
    assert got.count == 0 and got.hist == [] and got.hash == 0
