"""Benchmark: maximal cliques per second and end-to-end MCE time on one MI355X.

One step = one full mce_run over a device-resident CSR graph: validation, k-core
peel, orientation, the induced-subgraph builds and every search launch, ending
with the count, histogram and hash on the host (the timed scope of
"Parallelizing Maximal Clique Enumeration on GPUs", section 4.1: counting plus
degeneracy preprocessing, graph already loaded). The default workload is the
largest configuration whose whole clique set is checked against the oracle:
the Chung-Lu graph on 500,000 vertices with 2,000 planted cliques (12,690,421
maximal cliques). Moon-Moser n = 45 is measured as well and reported in
`detail.moon_moser45`.

Prints one JSON line. Besides the metric it reports:
  roofline      the dominant kernel of a step (the single launch with the largest
                time, from HIP events recorded on the engine's stream around every
                phase and launch): its algorithmic work per launch over its
                average launch time, against the peak of the unit that bounds it
                (int32 vector lane-ops for the search kernels, HBM bytes for the
                others); `traffic` is the HBM bytes of that kernel per launch from
                the committed rocprofv3 counter summary, when the sources it was
                taken on are the current ones.
  detail.kernels    every launch of a step the same way, with HBM and LDS
                fractions where counters exist.
  detail.cu_load    per search launch, per compute unit (section 4.3 measures
                load per SM): busy share and the max/mean of the per-CU load.
  cpu_baseline  the oracle (single-threaded C Bron-Kerbosch-Tomita) run over the
                subtree roots by one process per host core, timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

NUM_CU = 256
CLOCK_HZ = 2.4e9
# MI355X int32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-ops/s
VALU_INT32_PEAK = NUM_CU * 4 * 16 * CLOCK_HZ
HBM_PEAK = 8.0e12                       # bytes/s
LDS_PEAK = 128 * NUM_CU * CLOCK_HZ      # bytes/s: 128 B per clock per CU
# algorithmic int32 lane-ops per counted unit
OPS_PER_PIVOT_WORD = 4      # 64-bit AND (2) + 64-bit popcount (2)
OPS_PER_BRANCH_WORD = 10    # P n N(v), X_P n N(v) (2 x 2) and the C, P, X_P updates (3 x 2)
OPS_PER_XX_TEST = 2         # one bit test (full subgraph)
OPS_PER_LEAF = 20           # one mix64 of the clique's hash sum
MICRO_SUB = 12              # sub-class index of the micro kernel (launch_sub)

DEFAULT_COUNTERS = os.path.join(ROOT, "profiles", "kernel_counters.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3,
                    help="workload index (default 3: Chung-Lu 500k + 2,000 planted cliques)")
    ap.add_argument("--sample", choices=["uniform", "heavy", "dense"], default=None,
                    help="run on the workload's seeded root sample (tests/golden/configs.json) instead of "
                         "the whole graph: the maximal cliques whose earliest vertex is a sampled root")
    ap.add_argument("--cap-ms", type=int, default=0,
                    help="time-capped whole-graph run: the search stops at this limit and the cliques found "
                         "by then are counted (partial: no parity)")
    ap.add_argument("--whole-chunks", type=int, default=0,
                    help="whole graph in this many pieces (mce_run_roots): the roots the oracle finishes within "
                         "its budget first, then the heavy roots packed by their estimated subtree sizes; each "
                         "piece prints its result as it ends (configurations with a light set in configs.json)")
    ap.add_argument("--chunk-cap-ms", type=int, default=150000, help="time limit of one piece (--whole-chunks)")
    ap.add_argument("--first-chunk", type=int, default=0, help="resume --whole-chunks at this piece")
    ap.add_argument("--level", type=int, choices=[1, 2], default=1,
                    help="first-level (1, default) or second-level (2) subtrees")
    ap.add_argument("--subgraph", choices=["auto", "partial", "full"], default="auto",
                    help="induced-subgraph encoding: the engine's choice by max degree / degeneracy (default), "
                         "P only, or P and X")
    ap.add_argument("--events", choices=["auto", "phase", "search"], default="auto",
                    help="events in the timed runs: around every phase and launch, or around the search "
                         "launches only (auto: search only for graphs whose run takes about a millisecond)")
    ap.add_argument("--serial", action="store_true",
                    help="sub-class launches one after another on one stream (default: overlapped)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the oracle baseline")
    ap.add_argument("--cpu-procs", type=int, default=0, help="oracle processes (0: min(16, host cores))")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the Moon-Moser 45 detail measurement")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration runs)")
    ap.add_argument("--counters-json", default=DEFAULT_COUNTERS)
    return ap.parse_args()


# ---------------------------------------------------------------- counters
# The source file that defines each kernel family; every family also compiles
# the shared device headers.
KERNEL_SOURCES = {"k_peel": "prep.hip", "k_validate": "prep.hip", "k_search_micro": "micro.hip",
                  "k_search": "search.hip", "k_build": "subgraph.hip", "k_forward_adj": "prep.hip"}
SHARED_HEADERS = ("mce_device.h", "mce_internal.h", "worklist.h")


def family(kernel):
    for k in sorted(KERNEL_SOURCES, key=len, reverse=True):
        if kernel.startswith(k):
            return k
    return None


def sources_hash(kernel):
    """SHA-256 prefix over the source files that define `kernel` (a row such as
    "k_build_micro+k_forward_adj" names several kernels) and every header they
    include: a counter summary taken on other sources is not used."""
    files = []
    for part in kernel.split("+"):
        fam = family(part)
        if fam is None:
            return None
        if KERNEL_SOURCES[fam] not in files:
            files.append(KERNEL_SOURCES[fam])
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "maximal_clique_enumeration_amd", "csrc")
    for name in tuple(files) + SHARED_HEADERS:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_counters(path, workload):
    """The committed rocprofv3 counter summary for this workload: {row key: {...}}
    for the kernels whose sources are unchanged since it was taken."""
    if not os.path.exists(path):
        return {}
    try:
        with open(path) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return {}
    rows = doc.get("workloads", {}).get(workload, {})
    return {k: v for k, v in rows.items() if v.get("sources_sha256_16") == sources_hash(k.split("#")[0])}


# ---------------------------------------------------------------- work per launch
def kernel_name(sub):
    if sub == MICRO_SUB:
        return "k_search_micro"
    w = 1 << (sub >> 1)
    return "k_search_w1" if w == 1 else f"k_search<{w}>"


def build_name(sub):
    if sub == MICRO_SUB:
        return "k_build_micro"
    w = 1 << (sub >> 1)
    # widths up to 8 build their P rows in a kernel of their own (with the forward adjacency)
    return f"k_build_head+k_build_prows+k_build_rows<{w}>" if w <= 8 else f"k_build_head+k_build_rows<{w}>"


def launch_ops(trace, launch):
    """Algorithmic int32 lane-ops of one search launch, from a counting run's
    per-wavefront counters: pivot AND+popcount per word, the branches' set
    operations, X_X bit tests, one mix64 per clique."""
    rs = [t for t in trace if t["launch"] == launch]
    pw = sum(t["pivot_words"] for t in rs)
    br = sum(t["branches"] for t in rs)
    xx = sum(t["xx_tests"] for t in rs)
    lv = sum(t["leaves"] for t in rs)
    don = sum(t["donations"] for t in rs)
    return pw, br, xx, lv, don


def search_ops(pw, br, xx, lv, don, width, micro):
    # the wavefront kernels hand a donated branch over untaken: add those back;
    # the micro kernel hands over frames whose branches are counted where taken
    branches = br + (0 if micro else don)
    return pw * OPS_PER_PIVOT_WORD + branches * width * OPS_PER_BRANCH_WORD + xx * OPS_PER_XX_TEST + lv * OPS_PER_LEAF


def peel_bytes(n, nnz):
    """The peel's algorithmic HBM bytes: every row read once when its vertex
    leaves (row bounds 4(n+1), entries 4 nnz), one degree decrement per entry
    (read and write, 8 nnz), core number and round written (8 n)."""
    return 4 * (n + 1) + 12 * nnz + 8 * n


def build_bytes(words):
    """A build's algorithmic HBM bytes: the table words it writes (its reads of
    CSR rows are gathers whose volume depends on the hub rows it probes)."""
    return 8 * words


# ---------------------------------------------------------------- per-CU load
def cu_load(trace, num_cu):
    """Per search launch: where its waves ran (hardware ids), the share of the
    chip's compute-unit time in which the CU's busiest wave held a task, and the
    largest per-CU load over the mean (section 4.3: the load of an SM is the
    most tree nodes any of its blocks visited)."""
    out = []
    for lid in sorted({t["launch"] for t in trace}):
        # (a wave that found the run already stopped returns before it records anything)
        rs = [t for t in trace if t["launch"] == lid and t["start_tick"]]
        if not rs:
            out.append({"launch": lid, "waves": 0, "cus_seen": 0, "cu_busy_frac": None, "wave_busy_frac": None,
                        "cu_mean_wave_busy_frac": None, "cu_load_max_over_mean": None, "span_ms": None})
            continue
        span = max(t["end_tick"] for t in rs) - min(t["start_tick"] for t in rs)
        per_cu = {}
        for t in rs:
            key = ((t["hw_location"] >> 32) & 0xF, (t["hw_location"] >> 8) & 0xFF)
            c = per_cu.setdefault(key, [0, 0, 0])
            c[0] = max(c[0], t["busy_ticks"])
            c[1] = max(c[1], t["nodes"])
            c[2] += t["busy_ticks"]
        loads = [c[1] for c in per_cu.values()]
        mean = sum(loads) / len(loads) if loads else 0
        waves_per_cu = len(rs) / max(1, len(per_cu))
        out.append({"launch": lid, "waves": len(rs), "cus_seen": len(per_cu),
                    "cu_busy_frac": sum(c[0] for c in per_cu.values()) / (num_cu * span) if span else None,
                    "wave_busy_frac": sum(t["busy_ticks"] for t in rs) / (len(rs) * span) if span else None,
                    "cu_mean_wave_busy_frac": (sum(c[2] for c in per_cu.values()) / (waves_per_cu * num_cu * span)
                                               if span else None),
                    "cu_load_max_over_mean": max(loads) / mean if mean else None,
                    "span_ms": None})
    return out


# ---------------------------------------------------------------- CPU baseline
_POOL = {}


def _pool_init(path, shm_name, n):
    import numpy as np
    from multiprocessing import shared_memory
    d = np.load(path)
    _POOL["g"] = (int(d["n"]), d["rp"], d["ci"])
    _POOL["shm"] = shared_memory.SharedMemory(name=shm_name)
    _POOL["rnd"] = np.ndarray((max(n, 1),), dtype=np.int32, buffer=_POOL["shm"].buf)


def _pool_chunk(roots):
    import numpy as np
    import oracle
    n, rp, ci = _POOL["g"]
    r = oracle.mce(n, rp, ci, roots=np.asarray(roots, np.int32), rnd=_POOL["rnd"][:n])
    return r.count, r.hash, r.hist, len(roots)


def _pool_ping(_):
    return os.getpid()


def cpu_baseline(g, budget_s, procs, roots=None):
    """The oracle on this host: its peel in this process, then its first-level
    subtrees (the whole graph, or the sampled roots) in interleaved chunks over
    `procs` processes, for at most about budget_s seconds. Reports cliques per
    second over the whole timed span and whether the sums equal the GPU's."""
    import multiprocessing as mp
    import tempfile
    from multiprocessing import shared_memory

    import numpy as np

    import oracle
    allr = np.arange(g.n, dtype=np.int32) if roots is None else np.asarray(roots, np.int32)
    tmp = tempfile.NamedTemporaryFile(suffix=".npz", delete=False)
    tmp.close()
    np.savez(tmp.name, n=np.int64(g.n), rp=g.row_ptr, ci=g.col_idx)
    shm = shared_memory.SharedMemory(create=True, size=max(g.n, 1) * 4)
    ctx = mp.get_context("spawn")   # fresh interpreters: nothing of this process's GPU state
    try:
        with ctx.Pool(procs, initializer=_pool_init, initargs=(tmp.name, shm.name, g.n)) as pool:
            pool.map(_pool_ping, range(procs))   # the workers are up and hold the graph
            t0 = time.perf_counter()
            _, rnd, _ = oracle.peel(g.n, g.row_ptr, g.col_idx)
            np.ndarray((max(g.n, 1),), dtype=np.int32, buffer=shm.buf)[:g.n] = rnd
            t_peel = time.perf_counter() - t0
            nchunks = min(allr.size, max(1, 64 * procs))
            chunks = [allr[j::nchunks] for j in range(nchunks)]
            pending, done = [], []
            it = iter(chunks)
            stop = False
            while True:
                while not stop and len(pending) < 2 * procs:
                    c = next(it, None)
                    if c is None:
                        stop = True
                        break
                    pending.append(pool.apply_async(_pool_chunk, (c,)))
                if not pending:
                    break
                pending[0].wait()
                still = []
                for a in pending:
                    if a.ready():
                        done.append(a.get())
                    else:
                        still.append(a)
                pending = still
                if time.perf_counter() - t0 > budget_s:
                    stop = True
            t_used = time.perf_counter() - t0
    finally:
        shm.close()
        shm.unlink()
        os.unlink(tmp.name)
    cnt = sum(d[0] for d in done)
    hsh = sum(d[1] for d in done) % (1 << 64)
    hl = max((len(d[2]) for d in done), default=0)
    hist = [sum(d[2][k] for d in done if k < len(d[2])) for k in range(hl)]
    nroots = sum(d[3] for d in done)
    whole = nroots == allr.size
    what = "whole graph" if roots is None else f"{allr.size} sampled roots"
    sample = (f"{what}: oracle peel ({t_peel:.1f} s, 1 process) + {nroots} of {allr.size} first-level subtrees "
              f"in {procs} processes, {t_used:.1f} s")
    return {"value": cnt / t_used, "unit": "maximal cliques/s", "cores": procs, "kind": "oracle",
            "sample": sample, "complete": whole, "key": (cnt, hsh, tuple(hist))}


# ---------------------------------------------------------------- GPU measurement
def measure(mce, torch, g, args, rp, ci, roots, events, steps, warmup, cap_ms=0):
    """Counting run (exact work per launch), then `steps` timed runs."""
    timeout = cap_ms if cap_ms else 100000
    if cap_ms:
        ref, cst, ctrace = None, None, []   # a stopped run's work is not the workload's: no counting run
    else:
        with mce.Engine(device=0, counters=True, timeout_ms=timeout, level=args.level,
                        subgraph=args.subgraph, overlap=not args.serial) as ecnt:
            ref = ecnt.run(rp, ci, roots=roots)
            cst = ecnt.stats()
            ctrace = ecnt.worker_trace()
    eng = mce.Engine(device=0, timeout_ms=timeout, level=args.level, subgraph=args.subgraph,
                     search_times=events == "search", phase_times=events == "phase", overlap=not args.serial)
    for _ in range(warmup):
        r = eng.run(rp, ci, roots=roots, partial_ok=bool(cap_ms))
        if not cap_ms and r.key() != ref.key():
            raise SystemExit("results differ between runs")
    torch.cuda.synchronize()
    # Each step is one mce_run, which returns after the device work completed;
    # the step's counters and event times are read after it, outside the clock.
    times, stats, results = [], [], []
    for _ in range(steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = eng.run(rp, ci, roots=roots, partial_ok=bool(cap_ms))
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        stats.append(eng.stats())
        results.append(r)
        if not cap_ms and r.key() != ref.key():
            raise SystemExit("results differ between steps")
    trace = eng.worker_trace()
    info = eng.graph_info()
    eng.close()
    if cap_ms:
        ref, cst = results[-1], stats[-1]
    return ref, cst, ctrace, times, stats, results, trace, info


def kernel_table(g, cst, ctrace, stats, events, counters, nnz):
    """Every launch of a step with its mean time (events) and roofline figures."""
    n_st = len(stats)
    mean = lambda key: sum(s[key] for s in stats) / n_st   # noqa: E731
    rows = []
    if events == "phase":
        # a split peel is two launches (the grid's, then the tail's): the events span both
        rows.append({"kernel": "k_peel+k_peel_tail" if stats[0].get("handover_round", -1) >= 0 else "k_peel",
                     "ms": mean("ms_peel"), "bound": "hbm", "algorithmic": peel_bytes(g.n, nnz), "unit": "B"})
        rows.append({"kernel": "k_validate_*", "ms": mean("ms_validate"), "bound": "hbm",
                     "algorithmic": 4 * (g.n + 1) + 4 * nnz, "unit": "B"})
    launches = stats[0]["launches"]
    for i in range(launches):
        sub = stats[0]["launch_sub"][i]
        micro = sub == MICRO_SUB
        width = 1 if micro else 1 << (sub >> 1)
        sms = sum(s["launch_search_ms"][i] for s in stats) / n_st
        pw, br, xx, lv, don = launch_ops(ctrace, i)
        rows.append({"kernel": kernel_name(sub), "launch": i, "roots": stats[0]["launch_roots"][i], "ms": sms,
                     "bound": "alu", "algorithmic": search_ops(pw, br, xx, lv, don, width, micro), "unit": "ops"})
        if events == "phase":
            bms = sum(s["launch_build_ms"][i] for s in stats) / n_st
            rows.append({"kernel": build_name(sub), "launch": i, "ms": bms, "bound": "hbm",
                         "algorithmic": build_bytes(stats[0]["launch_words"][i]), "unit": "B"})
    for r in rows:
        sec = r["ms"] / 1e3
        if sec <= 0:
            r["frac"] = None
            continue
        if r["bound"] == "alu":
            r["achieved"] = r["algorithmic"] / sec / 1e12
            r["peak"] = VALU_INT32_PEAK / 1e12
            r["frac"] = r["algorithmic"] / sec / VALU_INT32_PEAK
        else:
            r["achieved"] = r["algorithmic"] / sec / 1e9
            r["peak"] = HBM_PEAK / 1e9
            r["frac"] = r["algorithmic"] / sec / HBM_PEAK
        # the counter passes run the launches in series (no split peel: one peel
        # launch, and the peel's order, whose sub-classes come in the same order)
        if "launch" not in r:
            ckey = "k_peel" if r["kernel"].startswith("k_peel") else r["kernel"]
        else:
            ckey = f'{r["kernel"]}#{r["launch"]}'
        c = counters.get(ckey)
        if c:
            traffic = c.get("fetch_bytes", 0) + c.get("write_bytes", 0)
            r["traffic"] = traffic
            r["hbm_frac"] = traffic / sec / HBM_PEAK
            if "lds_bytes" in c:
                # LDS bytes moved (SQ_INSTS_LDS_{LOAD,STORE,ATOMIC}_BANDWIDTH, 64-byte units)
                r["lds_bytes"] = c["lds_bytes"]
                r["lds_frac"] = c["lds_bytes"] / sec / LDS_PEAK
            if "sq_insts_valu" in c:
                # a wave64 VALU instruction holds a 16-lane SIMD for 4 cycles
                r["valu_issue_frac"] = c["sq_insts_valu"] * 4 / (NUM_CU * 4 * CLOCK_HZ * sec)
            if "sq_insts_salu" in c:
                # one scalar instruction per CU and cycle
                r["salu_issue_frac"] = c["sq_insts_salu"] / (NUM_CU * CLOCK_HZ * sec)
    return rows


def roofline_of(rows):
    top = max(rows, key=lambda r: r["ms"])
    unit = "Tops/s (int32 vector lane-ops)" if top["bound"] == "alu" else "GB/s"
    out = {"bound": top["bound"], "achieved": top.get("achieved"), "peak": top.get("peak"), "unit": unit,
           "frac": top.get("frac"), "traffic": top.get("traffic"), "kernel": top["kernel"],
           "launch_ms": top["ms"], "algorithmic_per_launch": top["algorithmic"]}
    for k in ("hbm_frac", "lds_frac", "valu_issue_frac", "salu_issue_frac", "launch"):
        if k in top:
            out[k] = top[k]
    return out


def whole_in_chunks(mce, torch, g, args, rp, ci, dev):
    """The whole graph as a sequence of mce_run_roots calls over disjoint root
    sets: first-level subtrees are independent (section 2.4), so the pieces'
    counts, histograms and hashes add up to the whole graph's. Piece 0 holds the
    roots whose subtrees the oracle finished within its budget (its sums are
    compared with the oracle's); the heavy roots follow, packed into pieces of
    about equal estimated size (Knuth's estimate, tests/golden/configs.json)."""
    import numpy as np
    with open(os.path.join(ROOT, "tests", "golden", "configs.json")) as f:
        gold = json.load(f)[str(args.config)]
    light = gold["light"]
    heavy = np.asarray(light["heavy_roots"], np.int64)
    est = np.asarray(light["heavy_est_nodes"], np.float64)
    k = max(1, args.whole_chunks - 1)
    order = np.argsort(-est, kind="stable")
    pieces = [[] for _ in range(k)]
    load = np.zeros(k)
    for i in order:                       # largest first, into the lightest piece
        j = int(np.argmin(load))
        pieces[j].append(int(heavy[i]))
        load[j] += est[i]
    mask = np.ones(g.n, bool)
    mask[heavy] = False
    plan = [np.flatnonzero(mask).astype(np.int32)] + [np.asarray(sorted(pc), np.int32) for pc in pieces if pc]
    results, times, completes = [], [], []
    total_cnt, total_hash, hist = 0, 0, []
    eng = mce.Engine(device=0, timeout_ms=args.chunk_cap_ms, level=args.level, subgraph=args.subgraph,
                     overlap=not args.serial)
    for i, roots in enumerate(plan):
        if i < args.first_chunk:
            continue
        rt = torch.from_numpy(roots).to(dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = eng.run(rp, ci, roots=rt, partial_ok=True)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        ok = None
        if i == 0:
            ok = (r.count, f"0x{r.hash:016x}", r.hist) == (light["count"], light["hash"], light["hist"])
        rec = {"piece": i, "roots": int(roots.size), "count": r.count, "hash": f"0x{r.hash:016x}",
               "complete": r.complete, "s": dt, "est_nodes": float(est[np.isin(heavy, roots)].sum()) if i else None,
               "matches_oracle": ok}
        print("bench: piece " + json.dumps(rec), file=sys.stderr, flush=True)
        results.append(rec)
        times.append(dt)
        completes.append(r.complete)
        total_cnt += r.count
        total_hash = (total_hash + r.hash) % (1 << 64)
        hist = [a + b for a, b in zip(hist + [0] * (len(r.hist) - len(hist)), r.hist + [0] * (len(hist) - len(r.hist)))]
    info = eng.graph_info()
    eng.close()
    return {"pieces": results, "count": total_cnt, "hash": f"0x{total_hash:016x}", "hist": hist,
            "seconds": sum(times), "complete": all(completes) and args.first_chunk == 0, "info": info,
            "npieces": len(plan)}


def workload_label(args):
    parts = [f"cfg{args.config}"]
    if args.sample:
        parts.append(args.sample)
    if args.level == 2:
        parts.append("l2")
    if args.subgraph != "auto":
        parts.append(args.subgraph)
    if args.cap_ms:
        parts.append(f"cap{args.cap_ms}")
    return "-".join(parts)


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
    print(f"bench: generating workload {args.config}", file=sys.stderr, flush=True)
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
    if args.whole_chunks:
        print(f"bench: whole graph in pieces", file=sys.stderr, flush=True)
        w = whole_in_chunks(mce, torch, g, args, rp, ci, dev)
        feas = None
        fpath = os.path.join(ROOT, "tests", "golden", "feasibility.json")
        if os.path.exists(fpath):
            with open(fpath) as f:
                feas = json.load(f).get(str(args.config))
        out = {"metric": "maximal cliques/sec and end-to-end MCE time per graph on 1 MI355X",
               "value": w["count"] / w["seconds"] if w["seconds"] else None, "unit": "maximal cliques/s",
               "n_gpus": 1, "steps": 1, "warmup": 0, "ms_per_step": w["seconds"] * 1e3,
               "higher_is_better": True, "scaling": "strong", "vs_baseline": None,
               "dtype": "u64 bitsets / int32 ids",
               "data": ("synthetic (seeded generator); whole graph as independent pieces of first-level "
                        "subtrees; parity: piece 0 against the oracle, the rest against its estimate only"),
               "config": {"workload": g.name, "n": g.n, "edges": g.m, "maximal_cliques": w["count"],
                          "complete": w["complete"], "pieces": w["npieces"], "hash": w["hash"],
                          "degeneracy": w["info"]["degeneracy"], "max_degree": w["info"]["max_degree"]},
               "detail": {"hist": w["hist"], "pieces": w["pieces"],
                          "oracle_estimate": ({"cliques": feas["total_cliques_est"],
                                               "cliques_se": feas["heavy_cliques_se"],
                                               "z": (w["count"] - feas["total_cliques_est"]) / feas["heavy_cliques_se"]
                                               if feas["heavy_cliques_se"] else None} if feas else None)},
               "roofline": None, "cpu_baseline": None}
        print(json.dumps(out), flush=True)
        return
    events = args.events
    if events == "auto":
        events = "search" if args.config in (0, 1) else "phase"
    print("bench: GPU runs", file=sys.stderr, flush=True)
    ref, cst, ctrace, times, stats, results, trace, info = measure(
        mce, torch, g, args, rp, ci, roots, events, args.steps, args.warmup, args.cap_ms)
    counters = load_counters(args.counters_json, workload_label(args))
    rows = kernel_table(g, cst, ctrace, stats, events, counters, g.nnz)
    total = sum(times)
    last = results[-1]
    count = last.count
    value = sum(r.count for r in results) / total
    complete = all(r.complete for r in results)
    balance = cu_load(trace, NUM_CU)
    for b in balance:
        b["span_ms"] = stats[-1]["launch_search_ms"][b["launch"]] if b["launch"] < stats[-1]["launches"] else None
    st = stats[-1]
    data = "synthetic (seeded generator; stands in for the public graphs the page measures)"
    if not complete:
        data += "; time-capped: the search stopped at the limit, partial count, no parity"
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
        "data": data,
        "config": {"workload": g.name, "n": g.n, "edges": g.m, "degeneracy": info["degeneracy"],
                   "max_degree": info["max_degree"], "maximal_cliques": count, "complete": complete,
                   "roots_started": info["roots_started"], "roots": info["roots"],
                   "subgraph": "full" if info["subgraph"] == mce.MCE_SUBGRAPH_FULL else "partial",
                   "parallelism": "single GPU: one search-tree node per lane (micro kernel) or one subtree "
                                  "per wavefront, branch requests between wavefronts",
                   "seed": args.seed, "sample": args.sample or "whole graph", "subtrees": f"level {args.level}",
                   "launches": "serial" if args.serial else "overlapped", "cap_ms": args.cap_ms or None},
        "roofline": roofline_of(rows),
        "detail": {"e2e_ms_min": min(times) * 1e3, "e2e_ms_median": sorted(times)[len(times) // 2] * 1e3,
                   "hash": hex(last.hash), "events": events,
                   "kernels": rows,
                   "ms_validate": st["ms_validate"], "ms_peel": st["ms_peel"], "ms_orient": st["ms_orient"],
                   "ms_build": st["ms_build"], "ms_search": st["ms_search"],
                   "nodes": cst["nodes"], "donations": st["donations"], "workers": st["workers"],
                   "search_steps": cst["steps"],
                   "lane_util": (cst["lane_steps"] / (64 * cst["steps"]) if cst["steps"] else None),
                   "peel_rounds": info["rounds"],
                   # block 0 of the peel: barrier waits, level passes, round work, total (ms)
                   "peel_ms_split": [t / st["tick_hz"] * 1e3 for t in st["peel_ticks"]],
                   "cu_load": balance,
                   "counters_profile": bool(counters),
                   # share of the search's wavefront cycles by activity (the counting run;
                   # the page's section 4.5 breakdown)
                   "activity": {k: v / max(1, sum(cst["act_cycles"].values())) for k, v in cst["act_cycles"].items()}},
    }
    if not args.no_extra and args.config == 3 and not args.sample and not args.cap_ms and args.level == 1:
        print("bench: Moon-Moser 45 detail", file=sys.stderr, flush=True)
        gm = mce_inputs.config_graph(1)
        mrp = torch.from_numpy(gm.row_ptr).to(dev)
        mci = torch.from_numpy(gm.col_idx).to(dev)
        sub = argparse.Namespace(**{**vars(args), "config": 1, "level": 1, "subgraph": "auto"})
        mref, mcst, mctrace, mt, mstats, _, _, _ = measure(mce, torch, gm, sub, mrp, mci, None, "search", 20, 3)
        mrows = kernel_table(gm, mcst, mctrace, mstats, "search", load_counters(args.counters_json, "cfg1"), gm.nnz)
        out["detail"]["moon_moser45"] = {"maximal_cliques": mref.count, "ms_per_step": sum(mt) / len(mt) * 1e3,
                                         "value": mref.count * len(mt) / sum(mt), "roofline": roofline_of(mrows)}
    if not args.no_cpu_baseline and not args.cap_ms:
        procs = args.cpu_procs or min(16, os.cpu_count() or 1)
        print(f"bench: oracle baseline on {procs} processes", file=sys.stderr, flush=True)
        cb = cpu_baseline(g, args.cpu_seconds, procs, roots_host)
        key = cb.pop("key")
        if cb["complete"]:
            cb["matches_gpu"] = key == ref.key()
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
