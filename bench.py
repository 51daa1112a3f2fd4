"""Benchmark: maximal cliques per second and end-to-end MCE time on one MI355X.

One step = one full mce_run over a device-resident CSR graph: validation, k-core
peel, orientation, and every search launch, ending with the count, histogram
and hash on the host (the timed scope of "Parallelizing Maximal Clique
Enumeration on GPUs", section 4.1: counting plus degeneracy preprocessing,
graph already loaded). The default workload is the Moon-Moser graph on 45
vertices (3^15 maximal cliques of size 15).

Prints one JSON line. Also reports:
  roofline      the search kernel's algorithmic integer/bitwise work per launch
                divided by its average launch time (HIP events around each launch
                on the engine's stream), against the chip's int32 VALU peak;
  cpu_baseline  the oracle (single-threaded CPU Bron-Kerbosch-Tomita) timed on a
                bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz int32 VALU lane-ops per second
VALU_INT32_PEAK = 256 * 64 * 2.4e9
# algorithmic int32 operations per counted unit (roofline)
OPS_PER_PIVOT_WORD = 4      # 64-bit AND (2) + 64-bit popcount (2 x v_bcnt)
OPS_PER_LEAF = 24           # one mix64 of the clique sum in 32-bit pieces
OPS_PER_XX_TEST = 16        # binary search step count ~ log2(degree), one compare each


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=1, help="workload index (default 1: Moon-Moser 45)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "search_traffic.json"))
    return ap.parse_args()


def cpu_baseline(g, budget_s):
    """The oracle on the same graph, repeated until the budget is used (one
    thread). Reports cliques per second over the whole sample."""
    import oracle
    reps, cliques, t_used = 0, 0, 0.0
    t0 = time.perf_counter()
    while True:
        r = oracle.mce(g.n, g.row_ptr, g.col_idx)
        reps += 1
        cliques += r.count
        t_used = time.perf_counter() - t0
        if t_used >= budget_s or reps >= 1000:
            break
    return {"value": cliques / t_used, "unit": "maximal cliques/s", "cores": 1, "kind": "oracle",
            "sample": f"whole graph x{reps} runs (ordering + enumeration), {t_used:.1f} s, 1 thread"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this engine runs on one GPU; --gpus must be 1 "
                          "(the design for more GPUs is described, not built)"}))
        sys.exit(2)
    import torch

    import maximal_clique_enumeration_amd as mce
    import mce_inputs

    if not mce.lib_built():
        from maximal_clique_enumeration_amd import build
        build.build()
    g = mce_inputs.config_graph(args.config, seed=args.seed)
    dev = torch.device("cuda", 0)
    rp = torch.from_numpy(g.row_ptr).to(dev)
    ci = torch.from_numpy(g.col_idx).to(dev)
    torch.cuda.synchronize()
    eng = mce.Engine(device=0, phase_times=True, timeout_ms=100000)
    ref = None
    for _ in range(args.warmup):
        ref = eng.run(rp, ci)
    torch.cuda.synchronize()
    times, search_ms, stats = [], [], []
    t_start = time.perf_counter()
    for _ in range(args.steps):
        t0 = time.perf_counter()
        r = eng.run(rp, ci)
        times.append(time.perf_counter() - t0)
        st = eng.stats()
        search_ms.append(st["ms_search"])
        stats.append(st)
        if ref is not None and r.key() != ref.key():
            raise SystemExit("results differ between steps")
        ref = r
    torch.cuda.synchronize()
    total = time.perf_counter() - t_start
    count = ref.count
    value = count * args.steps / total
    st = stats[-1]
    avg_search_s = sum(search_ms) / len(search_ms) / 1e3
    ops = (st["pivot_words"] * OPS_PER_PIVOT_WORD + st["leaves"] * OPS_PER_LEAF
           + st["xx_tests"] * OPS_PER_XX_TEST)
    achieved = ops / avg_search_s if avg_search_s > 0 else 0.0
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f)
            if tj.get("config") == args.config:
                traffic = tj.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    roofline = {"bound": "alu", "achieved": achieved / 1e12, "peak": VALU_INT32_PEAK / 1e12,
                "unit": "Tops/s (int32 VALU lane-ops)", "frac": achieved / VALU_INT32_PEAK,
                "traffic": traffic, "kernel": "k_search (search launch)",
                "search_ms": avg_search_s * 1e3, "ops_per_launch": ops}
    info = eng.graph_info()
    out = {
        "metric": "maximal cliques/sec and end-to-end MCE time per graph on 1 MI355X",
        "value": value,
        "unit": "maximal cliques/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "u64 bitsets / int32 ids",
        "data": "synthetic",
        "config": {"workload": g.name, "n": g.n, "edges": g.m, "degeneracy": info["degeneracy"],
                   "max_degree": info["max_degree"], "maximal_cliques": count,
                   "parallelism": "single GPU, one wavefront per subtree + worker list",
                   "seed": args.seed},
        "roofline": roofline,
        "detail": {"e2e_ms_min": min(times) * 1e3, "e2e_ms_median": sorted(times)[len(times) // 2] * 1e3,
                   "nodes": st["nodes"], "donations": st["donations"], "workers": st["workers"],
                   "busy_frac": (st["busy_ticks"] / (st["workers"] * st["kernel_ticks"])
                                 if st["workers"] and st["kernel_ticks"] else None),
                   "max_over_avg_nodes": (st["max_nodes"] / (st["nodes"] / st["workers"])
                                          if st["nodes"] and st["workers"] else None),
                   "ms_validate": st["ms_validate"], "ms_peel": st["ms_peel"],
                   "ms_orient": st["ms_orient"], "hash": hex(ref.hash)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(g, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    eng.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
