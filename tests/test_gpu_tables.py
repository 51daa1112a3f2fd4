"""GPU: the induced subgraphs the build writes (section 3.4), word for word.

End-to-end parity shows the build right wherever a wrong bit would change the
cliques found; a wrong row that changes only the search's speed (a pivot that
is not the maximiser, say) would go unseen there. Here every sampled root's
table, read back with mce_root_table, must equal the oracle's independent
encoding of the same root (oracle.root_table: adjacency looked up pair by pair
in the CSR), in the width and form the engine chose: micro tables (with their
X columns), and wide tables of widths 1 to 32 words, full and partial.
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
GRAPHS = {
    "er2000": lambda: mi.config_graph(0),
    "chung_lu_planted": lambda: mi.chung_lu(20000, 12.0, 2.3, None, 3, planted=40, planted_min=10, planted_max=30),
    "hub_clique": lambda: mi.hub_clique(700, 4, 3000, 0.7, 12, 700),
    "hub_clique_110": lambda: mi.hub_clique(110, 4, 3000, 0.7, 12, 110),
    "hub_clique_1100": lambda: mi.hub_clique(1100, 4, 3000, 0.7, 12, 1100),
    # more vertices than the peel's tail takes: the search (and these tables)
    # take the hand-over order, built while the tail runs
    "chung_lu_100k": lambda: mi.chung_lu(100000, 12.0, 2.3, None, 3, planted=40, planted_min=10, planted_max=30),
}


def handover_order(g, rnd, r0):
    """The search's vertex ranks after a split peel at round r0 (compared like
    rounds, then id): a vertex gone before r0 keeps its round; a vertex still
    present gets r0 + its number of neighbours still present."""
    src = np.repeat(np.arange(g.n), np.diff(g.row_ptr))
    tail = rnd >= r0
    live = np.bincount(src, weights=tail[g.col_idx] & tail[src], minlength=g.n).astype(np.int64)
    return np.where(tail, r0 + live, rnd).astype(np.int32)


def roots_to_check(g, rnd, k=250, seed=5):
    src = np.repeat(np.arange(g.n), np.diff(g.row_ptr))
    lat = (rnd[g.col_idx] > rnd[src]) | ((rnd[g.col_idx] == rnd[src]) & (g.col_idx > src))
    P = np.bincount(src, weights=lat, minlength=g.n).astype(np.int64)
    X = np.diff(g.row_ptr) - P
    rng = np.random.default_rng(seed)
    some = rng.choice(g.n, size=min(k, g.n), replace=False)
    widest = np.argsort(-P, kind="stable")[:20]
    most_x = np.argsort(-X, kind="stable")[:20]
    return sorted(set(int(v) for v in np.concatenate([some, widest, most_x]))), P, X


@pytest.mark.parametrize("subgraph", ["partial", "full"])
@pytest.mark.parametrize("name", sorted(GRAPHS))
def test_tables_equal_the_oracle_encoding(name, subgraph):
    g = GRAPHS[name]()
    print(f"case {name} subgraph={subgraph}", flush=True)
    rp = torch.from_numpy(g.row_ptr).to(DEV)
    ci = torch.from_numpy(g.col_idx).to(DEV)
    _, rnd, _ = oracle.peel(g.n, g.row_ptr, g.col_idx)
    seen = set()
    with mce.Engine(device=0, timeout_ms=60000, subgraph=subgraph) as e:
        got_all = e.run(rp, ci)
        want_all = oracle.mce(g.n, g.row_ptr, g.col_idx)
        assert got_all.key() == want_all.key()
        r0 = e.stats()["handover_round"]
        if r0 >= 0:   # the search took the hand-over order
            print(f"  hand-over at round {r0}: {int((rnd >= r0).sum())} vertices left", flush=True)
            rnd = handover_order(g, rnd, r0)
        roots, P, X = roots_to_check(g, rnd)
        for root in roots:
            t = e.root_table(root)
            if P[root] == 0:
                assert t is None, root   # no later neighbour: no table
                continue
            words, form = t
            W, micro, full = form & 0xFF, (form >> 8) & 1 == 1, (form >> 9) & 1 == 1
            p, x = int(P[root]), int(X[root])
            # the engine's routing: micro tables exactly for |P|, |X| <= 64, else the
            # narrowest width that holds P, in the run's subgraph form
            assert micro == (p <= 64 and x <= 64), (root, p, x)
            if not micro:
                assert 64 * W >= p and (W == 1 or 32 * W < p), (root, p, W)
                assert full == (subgraph == "full"), (root, form)
            want = oracle.root_table(g.n, g.row_ptr, g.col_idx, rnd, root, W, micro, full)
            assert len(words) == len(want), (root, len(words), len(want))
            if (p + x) % 2:   # the last id word's high half is padding
                words = words.copy()
                words[-1] &= np.uint64(0xFFFFFFFF)
            bad = np.nonzero(words != want)[0]
            assert bad.size == 0, (root, p, x, form, bad[:8].tolist())
            seen.add((W, micro, full))
    print(f"  forms checked: {sorted(seen)}", flush=True)
    assert seen, "no table was checked"
