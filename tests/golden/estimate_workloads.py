"""Sizes the workload configurations before anyone enumerates them whole.

For every first-level subtree root ("Parallelizing Maximal Clique Enumeration on
GPUs", section 2.4, Algorithm 3) the oracle searches the subtree exactly if it
takes at most LIGHT_BUDGET search-tree nodes (oracle.mce_each). The subtrees
that exceed it are estimated with Knuth's random probes (oracle.knuth, WALKS
walks each): node count (calls of Algorithm 2) and maximal cliques, each with
its standard error. The sums give the predicted clique count of the whole
graph and the oracle's predicted single-core time (nodes over its measured
node rate). Only the oracle runs here; the result goes to
tests/golden/feasibility.json.

Knuth's estimate is unbiased but heavy-tailed: a few walks of a deep subtree
can miss its bulk, so the standard errors are lower bounds on the real
uncertainty. The exact configurations (0, 1, 3) serve as checks of the method.

Run from the repository root:
    python tests/golden/estimate_workloads.py [config ...]
    python tests/golden/estimate_workloads.py --check 3 5000
The second form is the check of the method: a configuration whose exact count is
known, with a low budget so that many subtrees are estimated (stored under
"<config>-check-<budget>").
"""
from __future__ import annotations

import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import mce_inputs as mi  # noqa: E402
import oracle  # noqa: E402

LIGHT_BUDGET = 200_000   # nodes searched exactly per root
WALKS = 64               # Knuth walks per heavy root
CHUNK = 4096             # roots per exact task
PROCS = min(8, os.cpu_count() or 1)

_G = {}


def _exact(chunk):
    g, rnd = _G["g"], _G["rnd"]
    t0 = time.process_time()
    nodes, cnt, hsh, done = oracle.mce_each(g.n, g.row_ptr, g.col_idx, chunk, LIGHT_BUDGET, rnd)
    return chunk, nodes, cnt, hsh, done, time.process_time() - t0


def _probe(args):
    root, seed = args
    g, rnd = _G["g"], _G["rnd"]
    t0 = time.process_time()
    e = oracle.knuth(g.n, g.row_ptr, g.col_idx, int(root), WALKS, seed=seed, rnd=rnd)
    return int(root), e, time.process_time() - t0


def split_counts(g, rnd):
    src = np.repeat(np.arange(g.n, dtype=np.int64), g.degrees())
    dst = g.col_idx.astype(np.int64)
    later = (rnd[dst] > rnd[src]) | ((rnd[dst] == rnd[src]) & (dst > src))
    p = np.bincount(src[later], minlength=g.n)
    return p, g.degrees() - p


def estimate(idx, light_budget=LIGHT_BUDGET):
    global LIGHT_BUDGET
    LIGHT_BUDGET = light_budget
    t_start = time.time()
    g = mi.config_graph(idx)
    _, rnd, d = oracle.peel(g.n, g.row_ptr, g.col_idx)
    p, x = split_counts(g, rnd)
    _G["g"], _G["rnd"] = g, rnd
    ctx = mp.get_context("fork")   # the workers share the graph (no GPU in this process)
    roots = np.arange(g.n, dtype=np.int32)
    # heavy candidates first, so the long chunks start early
    order = roots[np.argsort(-(p.astype(np.int64) * (x + p)), kind="stable")]
    chunks = [order[i::max(1, g.n // CHUNK)] for i in range(max(1, g.n // CHUNK))]
    nodes = np.zeros(g.n, np.int64)
    cnt = np.zeros(g.n, np.uint64)
    hsh = np.zeros(g.n, np.uint64)
    done = np.zeros(g.n, np.uint8)
    cpu_exact = 0.0
    with ctx.Pool(PROCS) as pool:
        for ch, nd, c, h, dn, sec in pool.imap_unordered(_exact, chunks):
            nodes[ch], cnt[ch], hsh[ch], done[ch] = nd, c, h, dn
            cpu_exact += sec
        heavy = np.flatnonzero(done == 0)
        print(f"cfg{idx}: exact pass {time.time() - t_start:.0f} s, {heavy.size} heavy roots", flush=True)
        probes = {}
        cpu_probe = 0.0
        for r, e, sec in pool.imap_unordered(_probe, [(int(r), 1000 + int(r)) for r in heavy]):
            probes[r] = e
            cpu_probe += sec
    light = done == 1
    exact_nodes = int(nodes[light].sum())
    rate = exact_nodes / cpu_exact if cpu_exact > 0 else None   # oracle nodes per CPU second (light roots)
    est_nodes = sum(e.nodes for e in probes.values())
    est_cl = sum(e.cliques for e in probes.values())
    se_nodes = sum(e.nodes_se ** 2 for e in probes.values()) ** 0.5
    se_cl = sum(e.cliques_se ** 2 for e in probes.values()) ** 0.5
    top = sorted(probes.items(), key=lambda kv: -kv[1].nodes)[:25]
    rec = {
        "config": idx, "name": g.name, "n": g.n, "m": g.m, "degeneracy": d,
        "max_p": int(p.max()), "max_x": int(x.max()),
        "light_budget": LIGHT_BUDGET, "walks": WALKS,
        "light_roots": int(light.sum()), "light_count": int(cnt[light].sum()),
        "light_hash": f"0x{int(hsh[light].sum(dtype=np.uint64)):016x}", "light_nodes": exact_nodes,
        "oracle_nodes_per_cpu_s": rate,
        "heavy_roots": int(heavy.size),
        "heavy_nodes_est": est_nodes, "heavy_nodes_se": se_nodes,
        "heavy_cliques_est": est_cl, "heavy_cliques_se": se_cl,
        "total_cliques_est": int(cnt[light].sum()) + est_cl,
        "total_nodes_est": exact_nodes + est_nodes,
        "oracle_core_seconds_est": (exact_nodes + est_nodes) / rate if rate else None,
        "heavy_with_p_ge_300": int((p[heavy] >= 300).sum()), "heavy_with_x_ge_10000": int((x[heavy] >= 10000).sum()),
        "roots_with_p_ge_300": int((p >= 300).sum()), "roots_with_x_ge_10000": int((x >= 10000).sum()),
        "largest_heavy": [{"root": r, "p": int(p[r]), "x": int(x[r]), "nodes": e.nodes, "nodes_se": e.nodes_se,
                           "cliques": e.cliques, "cliques_se": e.cliques_se, "max_depth": e.max_depth}
                          for r, e in top],
        "cpu_seconds": {"exact": round(cpu_exact, 1), "probes": round(cpu_probe, 1),
                        "wall": round(time.time() - t_start, 1), "processes": PROCS},
    }
    return rec


def main():
    path = os.path.join(HERE, "feasibility.json")
    out = {}
    if os.path.exists(path):
        with open(path) as f:
            out = json.load(f)
    if sys.argv[1:2] == ["--check"]:
        idx, budget = int(sys.argv[2]), int(sys.argv[3])
        jobs = [(f"{idx}-check-{budget}", idx, budget)]
    else:
        jobs = [(str(i), i, LIGHT_BUDGET) for i in ([int(a) for a in sys.argv[1:]] or [3, 2, 4])]
    for key, idx, budget in jobs:
        rec = estimate(idx, budget)
        out[key] = rec
        print(json.dumps({k: v for k, v in rec.items() if k != "largest_heavy"}), flush=True)
        with open(path, "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
