"""Per-activity cycle breakdown of the search kernels ("Parallelizing Maximal
Clique Enumeration on GPUs", section 4.5 and Figure 5: cycles per block and
activity from clock reads). With MCE_FLAG_COUNTERS the counting instances of the
micro, width-1 and wide search kernels charge every cycle of every wavefront to
one activity; they must still find exactly the oracle's cliques."""
import pytest

import mce_inputs as mi
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # pragma: no cover - CPU-only runs deselect these
    pytest.skip("needs a GPU", allow_module_level=True)

import maximal_clique_enumeration_amd as mce  # noqa: E402

DEV = torch.device("cuda", 0)
_WANT = {}


def want_of(i, g):
    if i not in _WANT:
        w = oracle.mce(g.n, g.row_ptr, g.col_idx)
        assert w.complete
        _WANT[i] = (w.count, w.hist, w.hash)
    return _WANT[i]

# micro subtrees (|P| <= 64), width-1 and widths 2 and 4 (|P| up to 129), X_X
# filters (hub rows), many small subtrees
GRAPHS = [mi.moon_moser(18), mi.random_small(150, 0.7, 3), mi.complete(130), mi.hub_clique(40, 3, 200, 0.5, 2, 5),
          mi.chung_lu(3000, 8.0, 2.3, None, 11)]

# engine options: which kernel instances and staging variants run
OPTIONS = {
    "micro": dict(),
    "width1-and-wide": dict(micro=False),
    "hbm-staging": dict(micro=False, hbm_staging=True),
    "partial": dict(micro=False, subgraph="partial"),
    "second-level": dict(level=2),
}


def run(e, g):
    rp = torch.from_numpy(g.row_ptr).to(DEV)
    ci = torch.from_numpy(g.col_idx).to(DEV)
    print(f"case {g.name} n={g.n} m={g.m}", flush=True)
    return e.run(rp, ci)


@pytest.mark.parametrize("opt", list(OPTIONS))
def test_counting_runs_keep_results_and_charge_every_cycle(opt):
    if not mce.lib_built():
        from maximal_clique_enumeration_amd import build
        build.build()
    ratios = []
    with mce.Engine(device=0, timeout_ms=20000, counters=True, **OPTIONS[opt]) as e:
        for i, g in enumerate(GRAPHS):
            got = run(e, g)
            assert (got.count, got.hist, got.hash) == want_of(i, g), g.name
            st = e.stats()
            act = st["act_cycles"]
            assert list(act) == list(mce.ACTIVITIES)
            assert all(v >= 0 for v in act.values()), act
            assert act["worker_list"] > 0 and act["task_start"] > 0, act
            if st["nodes"] > 0:
                assert act["pivot"] > 0 and act["set_ops"] > 0 and act["cliques"] > 0, act
            # the cycles cover the wavefronts' whole runs: against their wall-clock
            # spans, the same clock ratio on every graph
            span = sum(r["end_tick"] - r["start_tick"] for r in e.worker_trace())
            assert span > 0
            ratios.append(sum(act.values()) / span)
    assert min(ratios) > 0.5 and max(ratios) < 3 * min(ratios), ratios


def test_plain_runs_charge_nothing():
    with mce.Engine(device=0, timeout_ms=20000) as e:
        for g in GRAPHS[:3]:
            run(e, g)
            assert not any(e.stats()["act_cycles"].values())


def test_search_times_record_the_search_alone():
    """MCE_FLAG_SEARCH_TIMES: events around the search launches only, the
    other phase times stay 0; MCE_FLAG_PHASE_TIMES gives all of them."""
    g = GRAPHS[0]
    with mce.Engine(device=0, timeout_ms=20000, search_times=True) as e:
        run(e, g)
        st = e.stats()
        assert st["ms_search"] > 0 and len(st["launch_search_ms"]) == st["launches"] >= 1
        assert abs(sum(st["launch_search_ms"]) - st["ms_search"]) < 1e-3
        assert st["ms_validate"] == st["ms_peel"] == st["ms_orient"] == st["ms_build"] == 0
    with mce.Engine(device=0, timeout_ms=20000, phase_times=True) as e:
        run(e, g)
        st = e.stats()
        assert min(st["ms_validate"], st["ms_peel"], st["ms_orient"], st["ms_build"], st["ms_search"]) > 0
