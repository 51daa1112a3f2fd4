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

Run from the repository root:  python tests/golden/make_configs.py
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


def later_counts(g, rnd):
    src = np.repeat(np.arange(g.n, dtype=np.int64), g.degrees())
    dst = g.col_idx.astype(np.int64)
    later = (rnd[dst] > rnd[src]) | ((rnd[dst] == rnd[src]) & (dst > src))
    return np.bincount(src[later], minlength=g.n)


def entry(res):
    return {"count": res.count, "hash": f"0x{res.hash:016x}", "hist": res.hist}


def main():
    out = {}
    path = os.path.join(HERE, "configs.json")
    if os.path.exists(path):
        with open(path) as f:
            out = json.load(f)
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
