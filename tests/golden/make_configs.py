"""Writes tests/golden/configs.json: the oracle's results on the five workload
configurations, for the GPU parity tests (test_gpu_configs.py).

Only the oracle computes the stored values. For each configuration the file
holds the SHA-256 of the generated CSR (so a change of the generator shows up as
a failing check, not as a silent mismatch) and:
  - whole-graph count, hash and histogram where the oracle finishes the whole
    graph in seconds to minutes (configurations 0, 1, 3);
  - otherwise the results on seeded root samples (the maximal cliques whose
    earliest vertex in the peel order is a sampled root, "Parallelizing Maximal
    Clique Enumeration on GPUs", section 2.4, Algorithm 3): uniformly drawn
    roots, and the roots with the largest later-neighbour sets, each kept only if
    the oracle finishes its subtree within a node budget (the test compares
    exactly the kept roots). The whole R-MAT and large Chung-Lu graphs have too
    many maximal cliques to enumerate in a test.

Configurations 2 and 4 also get, with --light (multi-process oracle runs):
  - "light": every root whose subtree the oracle finishes within LIGHT_BUDGET
    nodes (stored as the list of the other, "heavy" roots), with the count,
    hash and histogram of their cliques: all of the graph but its dense core;
  - "dense" (with --dense, after --light): heavy roots whose subtrees the
    oracle finishes within DENSE_BUDGET nodes, the largest |P| first. The
    candidates are the DENSE_TRY heavy roots of smallest estimated size: a
    single root's Knuth estimate from a few walks is far too low more often than
    not (the bulk of a heavy subtree sits on rare paths), so it only orders
    the candidates, and the oracle decides.

Run from the repository root:  python tests/golden/make_configs.py [config ...]
                               python tests/golden/make_configs.py --light 2 4
                               python tests/golden/make_configs.py --dense 2 4
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import mce_inputs as mi  # noqa: E402
import oracle  # noqa: E402

WHOLE = (0, 1, 3)
SAMPLED = (2, 4)
N_UNIFORM = 3000          # uniformly drawn roots per sampled configuration
UNIFORM_BUDGET = 200_000  # oracle search-tree nodes allowed per uniform root
HEAVY_POOL = 20_000       # the roots of largest |P| ...
N_HEAVY_TRY = 150         # ... of which this many, evenly spaced from the largest down, are tried
N_HEAVY_KEEP = 60         # heavy roots kept
HEAVY_BUDGET = 1_000_000  # oracle search-tree nodes allowed per heavy root
LIGHT_BUDGET = 200_000    # nodes per root of the "light" set
DENSE_BUDGET = 2_000_000  # nodes per root of the "dense" sample
DENSE_TRY = 800           # heavy roots tried for it
DENSE_KEEP = 40           # dense roots kept
DENSE_WALKS = 16          # Knuth walks per dense candidate
PROCS = min(8, os.cpu_count() or 1)
_G = {}


def later_counts(g, rnd):
    src = np.repeat(np.arange(g.n, dtype=np.int64), g.degrees())
    dst = g.col_idx.astype(np.int64)
    later = (rnd[dst] > rnd[src]) | ((rnd[dst] == rnd[src]) & (dst > src))
    return np.bincount(src[later], minlength=g.n)


def entry(res):
    return {"count": res.count, "hash": f"0x{res.hash:016x}", "hist": res.hist}


def _each(args):
    roots, budget = args
    g, rnd = _G["g"], _G["rnd"]
    nodes, _, _, done = oracle.mce_each(g.n, g.row_ptr, g.col_idx, roots, budget, rnd)
    return roots, nodes, done


def _sum(roots):
    g, rnd = _G["g"], _G["rnd"]
    r = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=roots, rnd=rnd)
    assert r.complete
    return r.count, r.hash, r.hist


def _probe(root):
    g, rnd = _G["g"], _G["rnd"]
    return root, oracle.knuth(g.n, g.row_ptr, g.col_idx, int(root), DENSE_WALKS, seed=7000 + int(root), rnd=rnd)


def add_up(parts):
    cnt = sum(c for c, _, _ in parts)
    hsh = sum(h for _, h, _ in parts) % (1 << 64)
    hl = max((len(h) for _, _, h in parts), default=0)
    hist = [sum(h[k] for _, _, h in parts if k < len(h)) for k in range(hl)]
    return {"count": cnt, "hash": f"0x{hsh:016x}", "hist": hist}


def light_set(idx, rec):
    """The light set (all roots but the heavy ones) and every heavy root's estimated size."""
    import multiprocessing as mp
    t0 = time.time()
    g = mi.config_graph(idx)
    assert g.sha256() == rec["sha256"]
    _, rnd, _ = oracle.peel(g.n, g.row_ptr, g.col_idx)
    _G["g"], _G["rnd"] = g, rnd
    p = later_counts(g, rnd)
    x = g.degrees() - p
    nch = max(1, g.n // 4096)
    order = np.argsort(-(p.astype(np.int64) * (x + p)), kind="stable").astype(np.int32)
    with mp.get_context("fork").Pool(PROCS) as pool:   # the workers share the graph
        done = np.zeros(g.n, bool)
        for roots, _, dn in pool.imap_unordered(_each, [(order[i::nch], LIGHT_BUDGET) for i in range(nch)]):
            done[roots] = dn.astype(bool)
        heavy = np.flatnonzero(~done).astype(np.int32)
        light = np.flatnonzero(done).astype(np.int32)
        print(idx, "light", light.size, "heavy", heavy.size, round(time.time() - t0), flush=True)
        parts = pool.map(_sum, [light[i::nch] for i in range(nch)])
        rec["light"] = {"budget": LIGHT_BUDGET, "roots": int(light.size), "heavy_roots": heavy.tolist(),
                        "max_p": int(p[light].max()), "max_x": int(x[light].max()),
                        "roots_x_ge_10000": int((x[light] >= 10000).sum()),
                        "roots_p_ge_300": int((p[light] >= 300).sum()), **add_up(parts)}
        print(idx, "light done", round(time.time() - t0), flush=True)
        # every heavy root's estimated subtree size (nodes), to plan whole-graph runs in pieces
        est = dict(pool.map(_probe, [int(r) for r in heavy]))
        rec["light"]["heavy_est_nodes"] = [round(est[int(r)].nodes) for r in heavy]


def dense_sample(idx, rec):
    """Heavy roots that the oracle finishes within DENSE_BUDGET nodes, the largest |P| first."""
    import multiprocessing as mp
    t0 = time.time()
    g = mi.config_graph(idx)
    assert g.sha256() == rec["sha256"]
    _, rnd, _ = oracle.peel(g.n, g.row_ptr, g.col_idx)
    _G["g"], _G["rnd"] = g, rnd
    p = later_counts(g, rnd)
    x = g.degrees() - p
    heavy = np.asarray(rec["light"]["heavy_roots"], np.int32)
    est = np.asarray(rec["light"]["heavy_est_nodes"], np.float64)
    cand = heavy[np.argsort(est, kind="stable")][:DENSE_TRY]
    with mp.get_context("fork").Pool(PROCS) as pool:
        kept = []
        for roots, nodes, dn in pool.imap_unordered(_each, [(np.array([r], np.int32), DENSE_BUDGET) for r in cand]):
            if dn[0]:
                kept.append(int(roots[0]))
        kept = sorted(kept, key=lambda r: -p[r])[:DENSE_KEEP]
        dense = np.array(sorted(kept), np.int32)
        parts = pool.map(_sum, [dense[i::PROCS] for i in range(PROCS) if dense[i::PROCS].size])
    rec["dense"] = {"budget": DENSE_BUDGET, "roots": dense.tolist(), "tried": int(cand.size),
                    "p_range": [int(p[dense].min()), int(p[dense].max())] if dense.size else None,
                    "x_range": [int(x[dense].min()), int(x[dense].max())] if dense.size else None,
                    **add_up(parts)}
    print(idx, "dense", dense.size, rec["dense"]["p_range"], rec["dense"]["x_range"], round(time.time() - t0),
          flush=True)


def main():
    out = {}
    path = os.path.join(HERE, "configs.json")
    if os.path.exists(path):
        with open(path) as f:
            out = json.load(f)
    if sys.argv[1:2] in (["--light"], ["--dense"]):
        for idx in [int(a) for a in sys.argv[2:]] or list(SAMPLED):
            (light_set if sys.argv[1] == "--light" else dense_sample)(idx, out[str(idx)])
            with open(path, "w") as f:
                json.dump(out, f, indent=1)
        return
    which = [int(a) for a in sys.argv[1:]] or list(WHOLE + SAMPLED)
    for idx in which:
        t0 = time.time()
        g = mi.config_graph(idx)
        rec = {"sha256": g.sha256(), "n": g.n, "m": g.m}
        _, rnd, d = oracle.peel(g.n, g.row_ptr, g.col_idx)
        rec["degeneracy"] = d
        if idx in WHOLE:
            r = oracle.mce(g.n, g.row_ptr, g.col_idx, rnd=rnd)
            assert r.complete
            rec["whole"] = entry(r)
        else:
            rng = np.random.default_rng(1000 + idx)
            draw = np.sort(rng.choice(g.n, size=N_UNIFORM, replace=False)).astype(np.int32)
            kept = [int(v) for v in draw
                    if oracle.mce(g.n, g.row_ptr, g.col_idx, roots=np.array([v], np.int32),
                                  node_budget=UNIFORM_BUDGET, rnd=rnd).complete]
            uni = np.array(kept, np.int32)
            r = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=uni, rnd=rnd)
            assert r.complete
            rec["uniform"] = {"roots": uni.tolist(), "drawn": int(draw.size), **entry(r)}
            print(idx, "uniform", uni.size, "of", draw.size, round(time.time() - t0, 1), flush=True)
            p = later_counts(g, rnd)
            # the very largest |P| sit in the dense core, whose subtrees exceed any
            # test budget: spread the candidates over the largest HEAVY_POOL
            pool = np.argsort(-p, kind="stable")[:HEAVY_POOL]
            cand = pool[np.linspace(0, pool.size - 1, min(N_HEAVY_TRY, pool.size)).astype(np.int64)]
            keep = []
            for v in cand:
                rv = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=np.array([v], np.int32),
                                node_budget=HEAVY_BUDGET, rnd=rnd)
                if rv.complete:
                    keep.append(int(v))
                if len(keep) >= N_HEAVY_KEEP:
                    break
            heavy = np.array(sorted(keep), np.int32)
            r = oracle.mce(g.n, g.row_ptr, g.col_idx, roots=heavy, rnd=rnd)
            assert r.complete
            rec["heavy"] = {"roots": heavy.tolist(), "max_p": int(p[heavy].max()) if len(heavy) else 0,
                            **entry(r)}
        rec["oracle_seconds"] = round(time.time() - t0, 1)
        out[str(idx)] = rec
        print(idx, {k: v for k, v in rec.items() if k not in ("uniform", "heavy")}, flush=True)
        with open(path, "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
