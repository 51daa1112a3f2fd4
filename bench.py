"""Benchmark: maximal cliques per second and end-to-end MCE time on one MI355X.

One step = one full mce_run over a device-resident CSR graph: validation, k-core
peel, orientation, the induced-subgraph builds and every search launch, ending
with the count, histogram and hash on the host (the timed scope of
"Parallelizing Maximal Clique Enumeration on GPUs", section 4.1: counting plus
degeneracy preprocessing, graph already loaded). The default workload is the
Moon-Moser graph on 45 vertices (3^15 maximal cliques of size 15).

Prints one JSON line. Besides the metric it reports:
  roofline      the search kernel's algorithmic integer/bitwise lane-ops per
                launch divided by its average launch time (HIP events around each
                search launch, recorded on the engine's stream), against the int32
                vector peak. The search tree does not depend on scheduling, so one
                counting run gives the exact work of every timed run.
  cpu_baseline  the oracle (single-threaded CPU Bron-Kerbosch-Tomita) timed on the
                same graph on this host.
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

# MI355X int32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-ops/s
VALU_INT32_PEAK = 256 * 4 * 16 * 2.4e9
# algorithmic int32 lane-ops per counted unit
OPS_PER_PIVOT_WORD = 4      # 64-bit AND (2) + 64-bit popcount (2)
OPS_PER_BRANCH_WORD = 10    # P n N(v), X_P n N(v) (2 x 2) and the C, P, X_P updates (3 x 2)
OPS_PER_XX_TEST = 2         # one bit test (full subgraph)
OPS_PER_LEAF = 20           # one mix64 of the clique's hash sum


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=1, help="workload index (default 1: Moon-Moser 45)")
    ap.add_argument("--sample", choices=["uniform", "heavy"], default=None,
                    help="run on the workload's seeded root sample (tests/golden/configs.json) instead of "
                         "the whole graph: the maximal cliques whose earliest vertex is a sampled root")
    ap.add_argument("--level", type=int, choices=[1, 2], default=1,
                    help="first-level (1, default) or second-level (2) subtrees")
    ap.add_argument("--subgraph", choices=["auto", "partial", "full"], default="auto",
                    help="induced-subgraph encoding: the engine's choice by max degree / degeneracy (default), "
                         "P only, or P and X")
    ap.add_argument("--balance", action="store_true",
                    help="add each search launch's load balance (from the per-wavefront trace)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration runs)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "search_traffic.json"))
    ap.add_argument("--counters-json", default=os.path.join(ROOT, "profiles", "search_counters.json"))
    return ap.parse_args()


KERNEL_SOURCES = {"k_search_micro": "micro.hip", "k_search_w1": "search.hip", "k_search": "search.hip"}


def kernel_source_hash(kernel):
    """SHA-256 prefix of the source file that defines `kernel` (profiles taken on
    another version of the kernel are not used)."""
    import hashlib
    path = os.path.join(ROOT, "maximal_clique_enumeration_amd", "csrc", KERNEL_SOURCES[kernel])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_profile(path, config, kernel):
    """A committed counter summary for this workload and the current kernel source, or None."""
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            tj = json.load(f)
    except (OSError, ValueError):
        return None
    if tj.get("config") != config or tj.get("kernel_family") != kernel:
        return None
    if tj.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return tj


def algorithmic_ops(st):
    w = st["pivot_words"] / st["pivot_rows"] if st["pivot_rows"] else 1.0
    # the wavefront kernels hand a donated branch over untaken: add those back;
    # the micro kernel hands over frames whose branches are counted where taken
    branches = st["branches"] + (st["donations"] if st["steps"] == 0 else 0)
    return (st["pivot_words"] * OPS_PER_PIVOT_WORD + branches * w * OPS_PER_BRANCH_WORD
            + st["xx_tests"] * OPS_PER_XX_TEST + st["leaves"] * OPS_PER_LEAF)


def cpu_baseline(g, budget_s, roots=None):
    """The oracle on this host, single-threaded, for about budget_s seconds: the
    whole graph repeated, or (root sample) its roots in chunks of 16, in order.
    Reports cliques per second over what it ran."""
    import oracle
    reps, cliques = 0, 0
    t0 = time.perf_counter()
    if roots is None:
        while True:
            r = oracle.mce(g.n, g.row_ptr, g.col_idx)
            reps += 1
            cliques += r.count
            t_used = time.perf_counter() - t0
            if t_used >= budget_s or reps >= 1000:
                break
        sample = f"whole graph x{reps} runs (ordering + enumeration), {t_used:.1f} s, 1 thread"
    else:
        import numpy as np
        _, rnd, _ = oracle.peel(g.n, g.row_ptr, g.col_idx)
        done = 0
        for i in range(0, len(roots), 16):
            chunk = np.asarray(roots[i:i + 16], np.int32)
            cliques += oracle.mce(g.n, g.row_ptr, g.col_idx, roots=chunk, rnd=rnd).count
            done += chunk.size
            if time.perf_counter() - t0 >= budget_s:
                break
        t_used = time.perf_counter() - t0
        sample = f"first {done} of {len(roots)} sampled roots (ordering + enumeration), {t_used:.1f} s, 1 thread"
    return {"value": cliques / t_used, "unit": "maximal cliques/s", "cores": 1, "kind": "oracle",
            "sample": sample}


def balance(trace):
    """Per search launch: the share of wavefront-time spent holding a task
    (busy ticks over waves x the launch's span), and the largest wavefront's node
    count over the mean (section 4.3's load measure)."""
    out = []
    for lid in sorted({t["launch"] for t in trace}):
        rs = [t for t in trace if t["launch"] == lid]
        span = max(t["end_tick"] for t in rs) - min(t["start_tick"] for t in rs)
        nodes = [t["nodes"] for t in rs]
        mean = sum(nodes) / len(nodes)
        out.append({"launch": lid, "waves": len(rs),
                    "busy_frac": sum(t["busy_ticks"] for t in rs) / (len(rs) * span) if span else None,
                    "max_over_mean_nodes": max(nodes) / mean if mean else None})
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this engine runs on one GPU; --gpus must be 1 "
                          "(the design for more GPUs is described, not built)"}))
        sys.exit(2)
    import torch

    import maximal_clique_enumeration_amd as mce
    import mce_inputs

    mce.load_library()   # raises if the HIP library is not built: no fallback
    g = mce_inputs.config_graph(args.config, seed=args.seed)
    dev = torch.device("cuda", 0)
    rp = torch.from_numpy(g.row_ptr).to(dev)
    ci = torch.from_numpy(g.col_idx).to(dev)
    roots_host, roots = None, None
    if args.sample:
        with open(os.path.join(ROOT, "tests", "golden", "configs.json")) as f:
            gold = json.load(f)[str(args.config)]
        if args.sample not in gold:
            raise SystemExit(f"workload {args.config} has no {args.sample} root sample")
        roots_host = gold[args.sample]["roots"]
        roots = torch.tensor(roots_host, dtype=torch.int32, device=dev)
    if args.calib_copy_mb:
        src = torch.empty(args.calib_copy_mb << 18, dtype=torch.int32, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
    torch.cuda.synchronize()

    # counting run: exact algorithmic work of the search (deterministic tree)
    with mce.Engine(device=0, counters=True, timeout_ms=100000, level=args.level, subgraph=args.subgraph) as ecnt:
        ref = ecnt.run(rp, ci, roots=roots)
        cst = ecnt.stats()
    ops = algorithmic_ops(cst)

    # the timed engine records events around the search launches only (the
    # roofline's kernel time); every event costs the stream a few microseconds,
    # so the per-phase times come from one more run after the clock stops
    eng = mce.Engine(device=0, search_times=True, timeout_ms=100000, level=args.level, subgraph=args.subgraph)
    for _ in range(args.warmup):
        r = eng.run(rp, ci, roots=roots)
        if r.key() != ref.key():
            raise SystemExit("results differ between runs")
    torch.cuda.synchronize()
    # Each step is one mce_run, which returns after the device work completed;
    # the step's counters and event times are read after it, outside the clock.
    times, search_ms, stats = [], [], []
    for _ in range(args.steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = eng.run(rp, ci, roots=roots)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        st = eng.stats()
        search_ms.append(st["ms_search"])
        stats.append(st)
        if r.key() != ref.key():
            raise SystemExit("results differ between steps")
    with mce.Engine(device=0, phase_times=True, timeout_ms=100000, level=args.level, subgraph=args.subgraph) as eph:
        for _ in range(2):   # the second: the engine's buffers exist
            eph.run(rp, ci, roots=roots)
        pst = eph.stats()
    total = sum(times)
    count = ref.count
    value = count * args.steps / total
    st = stats[-1]
    avg_search_s = sum(search_ms) / len(search_ms) / 1e3
    launches = max(1, st["launches"])
    achieved = ops / avg_search_s if avg_search_s > 0 else 0.0
    kernel = "k_search_micro" if st["steps"] > 0 and launches == 1 else "k_search_w1"
    default_workload = args.sample is None and args.level == 1 and args.subgraph == "auto"
    tj = load_profile(args.traffic_json, args.config, kernel) if default_workload else None
    traffic = tj.get("bytes_per_launch") if tj else None
    roofline = {"bound": "alu", "achieved": achieved / 1e12, "peak": VALU_INT32_PEAK / 1e12,
                "unit": "Tops/s (int32 vector lane-ops)", "frac": achieved / VALU_INT32_PEAK,
                "traffic": traffic, "kernel": kernel,
                "search_ms_per_step": avg_search_s * 1e3, "launches_per_step": launches,
                "ops_per_step": ops}
    cj = load_profile(args.counters_json, args.config, kernel) if default_workload else None
    if cj and avg_search_s > 0:
        # VALU issue: each wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles
        simd_cycles = 256 * 4 * 2.4e9 * avg_search_s
        roofline["valu_issue_frac"] = cj["sq_insts_valu_per_launch"] * 4 / simd_cycles
        roofline["salu_issue_frac"] = cj["sq_insts_salu_per_launch"] / (256 * 2.4e9 * avg_search_s)
    info = eng.graph_info()
    busy = (st["busy_ticks"] / (st["workers"] * st["kernel_ticks"])
            if st["workers"] and st["kernel_ticks"] else None)
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
                   "subgraph": "full" if info["subgraph"] == mce.MCE_SUBGRAPH_FULL else "partial",
                   "parallelism": "single GPU: one search-tree node per lane (micro kernel), frame stacks "
                                  "per wavefront, branch requests between wavefronts",
                   "seed": args.seed, "roots": args.sample or "all", "subtrees": f"level {args.level}"},
        "roofline": roofline,
        "detail": {"e2e_ms_min": min(times) * 1e3, "e2e_ms_median": sorted(times)[len(times) // 2] * 1e3,
                   "nodes": st["nodes"], "donations": st["donations"], "workers": st["workers"],
                   "steps": st["steps"], "lane_util": (st["lane_steps"] / (64 * st["steps"]) if st["steps"] else None),
                   "busy_frac": busy,
                   "max_over_avg_nodes": (st["max_nodes"] / (st["nodes"] / st["workers"])
                                          if st["nodes"] and st["workers"] else None),
                   # phase times of one run with an event around every phase (outside the clock)
                   "ms_validate": pst["ms_validate"], "ms_peel": pst["ms_peel"],
                   "ms_orient": pst["ms_orient"], "ms_build": pst["ms_build"],
                   "pivot_rows": cst["pivot_rows"], "branches": cst["branches"],
                   "xx_tests": cst["xx_tests"], "leaves": cst["leaves"], "hash": hex(ref.hash),
                   # share of the search's wavefront cycles by activity (the counting run;
                   # the page's section 4.5 breakdown)
                   "activity": {k: v / max(1, sum(cst["act_cycles"].values())) for k, v in cst["act_cycles"].items()}},
    }
    if args.balance:
        out["detail"]["balance"] = balance(eng.worker_trace())
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(g, args.cpu_seconds, roots_host)
    else:
        out["cpu_baseline"] = None
    eng.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
