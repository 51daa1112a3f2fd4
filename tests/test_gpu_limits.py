"""GPU: the search's own time limit, and what a stopped run leaves behind.

A run whose search passes mce_config.timeout_ms stops at the next deadline
check of every wavefront (the waves exit normally: nothing is killed), returns
MCE_ERR_TIMEOUT and keeps the maximal cliques found before the stop, marked
incomplete. The engine must stay usable: the next run on it is exact.

Moon-Moser n = 45 with one wavefront and no worker list takes about a second of
search, so a 1 ms limit (counted from the start of the peel) stops it in the
search; a 6-vertex graph finishes before its first deadline check.
"""
import json
import os

import pytest

import mce_inputs as mi
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # pragma: no cover - CPU-only runs deselect these
    pytest.skip("needs a GPU", allow_module_level=True)

import maximal_clique_enumeration_amd as mce  # noqa: E402

DEV = torch.device("cuda", 0)
HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "configs.json")) as f:
    MM45 = json.load(f)["1"]["whole"]   # the oracle's values for Moon-Moser n = 45


def on_gpu(g):
    return torch.from_numpy(g.row_ptr).to(DEV), torch.from_numpy(g.col_idx).to(DEV)


@pytest.mark.parametrize("micro", [True, False])
def test_search_stops_at_its_deadline_and_keeps_partial_results(micro):
    g = mi.moon_moser(45)
    rp, ci = on_gpu(g)
    print(f"case moon_moser45 micro={micro} timeout 1 ms, one wave", flush=True)
    with mce.Engine(device=0, timeout_ms=1, max_workers=1, worker_list=False, micro=micro) as e:
        with pytest.raises(mce.MceError) as ex:
            e.run(rp, ci)
        assert ex.value.status == mce.MCE_ERR_TIMEOUT
        part = e.result()
        info = e.graph_info()
        assert not part.complete and info["complete"] == 0
        assert 0 < info["roots_started"] <= g.n
        # every clique found is a maximal clique of size 15, and some are missing
        assert part.count == sum(part.hist) < MM45["count"]
        assert all(c == 0 for k, c in enumerate(part.hist) if k != 15)
        # the same run through partial_ok returns the partial sums instead of raising
        again = e.run(rp, ci, partial_ok=True)
        assert not again.complete and again.count < MM45["count"]

        # the engine is reusable: a graph that finishes before the first check is exact
        small = mi.fig1a()
        srp, sci = on_gpu(small)
        got = e.run(srp, sci)
        want = oracle.mce(small.n, small.row_ptr, small.col_idx)
        assert got.complete and e.graph_info()["complete"] == 1
        assert got.key() == want.key()


def test_full_run_after_a_stopped_one():
    """A stopped run leaves no state behind that a later run on another engine
    (same device buffers reused by the allocator) could pick up."""
    g = mi.moon_moser(45)
    rp, ci = on_gpu(g)
    with mce.Engine(device=0, timeout_ms=1, max_workers=4) as e:
        with pytest.raises(mce.MceError):
            e.run(rp, ci)
    with mce.Engine(device=0, timeout_ms=60000) as e:
        got = e.run(rp, ci)
        assert got.complete
        assert got.count == MM45["count"] and got.hist == MM45["hist"]
        assert f"0x{got.hash:016x}" == MM45["hash"]
        assert e.graph_info()["roots_started"] == g.n


def test_micro_stack_grows_after_an_overflow():
    """A micro frame stack too small for the search aborts the attempt; the
    engine runs the whole graph again with four times the frames, keeps that
    size for later runs, and the result is exact."""
    g = mi.moon_moser(45)
    rp, ci = on_gpu(g)
    print("case moon_moser45 micro_stack_frames=64, one wave", flush=True)
    with mce.Engine(device=0, timeout_ms=60000, max_workers=1, worker_list=False,
                    micro_stack_frames=64) as e:
        for _ in range(2):
            got = e.run(rp, ci)
            st = e.stats()
            assert got.complete
            assert got.count == MM45["count"] and got.hist == MM45["hist"]
            assert f"0x{got.hash:016x}" == MM45["hash"]
            assert 64 < st["micro_stack_cap"] <= 1 << 20
            assert st["micro_stack_cap"] & (st["micro_stack_cap"] - 1) == 0
        grown = st["micro_stack_cap"]
        # the grown size stays: a third run starts with it
        e.run(rp, ci)
        assert e.stats()["micro_stack_cap"] == grown
