"""CPU model of the worker-list protocol (the page's section 3.3; csrc/worklist.h).

The GPU kernels pass work between wavefronts through one request word per
wave (per slot), a wake flag per wave, a mailbox, an active count and a
shared root counter, using only atomic operations on single words. This model
runs the same protocol with each wavefront as a coroutine whose every shared
access is one atomic step, interleaved by a seeded random scheduler over
thousands of schedules, and checks what the kernels rely on:
  - every search-tree node of every subtree is processed exactly once (no
    donated branch is lost or taken twice);
  - the launch ends: every wave leaves, and only after all work is done;
  - the active count never goes below zero and ends at zero;
  - a wake flag is only written with a task while its owner waits for one;
  - no request is overwritten before it is answered.
Planted mistakes (each a bug the kernels avoid)
break these invariants in the model.
It models the protocol's logic in sequentially consistent steps (the kernels
keep each wave's order with waits for store completion between the steps that
depend on it); it is not a model of the memory system.
"""
import random

import pytest

OPEN, CLOSED = 0, -1
TASK, RETRY, EXIT = 1, 2, 3


class Launch:
    def __init__(self, roots, nwaves, nslots, rng):
        self.roots = list(roots)          # nodes in each first-level subtree
        self.root_ctr = 0
        self.n_active = 0
        self.req = [[CLOSED] * nslots for _ in range(nwaves)]
        self.flag = [0] * nwaves
        self.mail = [None] * nwaves
        self.open = set()                 # the open-request hint (a bitmap on the GPU)
        self.waiting = [False] * nwaves   # the model's own record: the wave waits on its flag
        self.processed = 0
        self.lost = 0                     # requests overwritten before they were answered
        self.nwaves, self.nslots, self.rng = nwaves, nslots, rng
        self.min_active = 0

    def add_active(self, d):
        self.n_active += d
        self.min_active = min(self.min_active, self.n_active)
        return self.n_active


def wave(L, w, plant=None):
    """One wavefront: phase 1 (shared root counter), then phase 2 (worker list).
    `plant` puts a known mistake into the protocol, for the tests that check
    that the model would see it."""
    L.add_active(1)                       # wl_join, before the first root is taken
    yield
    closed = True
    task = None
    while True:
        if task is None:
            idx = L.root_ctr              # take_root: one fetch-and-add
            L.root_ctr += 1
            yield
            if idx < len(L.roots):
                task = L.roots[idx]
                for _ in range(4):        # the subtree's table is built
                    yield
            else:
                # wl_idle: close the request slots (refusing what raced in)
                for k in range(L.nslots):
                    old = L.req[w][k]
                    L.req[w][k] = CLOSED
                    yield
                    if old not in (OPEN, CLOSED):
                        L.flag[old - 1] = RETRY
                        yield
                L.open.discard(w)
                L.flag[w] = 0
                yield
                left = L.add_active(-1)
                yield
                got = False
                if left > 0 and L.nwaves > 1:
                    L.waiting[w] = True
                    while True:
                        if L.flag[w] == EXIT:
                            break
                        cands = sorted(L.open - {w})
                        yield
                        if not cands:
                            continue
                        v = L.rng.choice(cands)
                        k = L.rng.randrange(L.nslots)
                        if L.req[v][k] != OPEN:
                            yield
                            continue
                        L.req[v][k] = w + 1   # compare-and-swap from OPEN (one atomic step)
                        yield
                        stop = False
                        while True:
                            a = L.flag[w]
                            yield
                            if a == TASK:
                                got = stop = True
                                break
                            if a == EXIT:
                                stop = True
                                break
                            if a == RETRY:
                                if plant == "plain_retry":
                                    yield                # mistake: a plain store consumes the refusal,
                                    L.flag[w] = 0        # and may erase an exit broadcast just written
                                elif L.flag[w] == RETRY:   # compare-and-swap RETRY -> 0
                                    L.flag[w] = 0
                                else:
                                    stop = True          # the exit broadcast replaced the refusal
                                yield
                                break
                        if stop:
                            break
                    L.waiting[w] = False
                if left <= 0:
                    for i in range(L.nwaves):
                        L.flag[i] = EXIT
                        yield
                if not got:
                    return
                task = L.mail[w]
                L.mail[w] = None
        # a task: reopen the request slots if they were closed, then search it
        if closed:
            for k in range(L.nslots):
                if L.req[w][k] not in (OPEN, CLOSED):
                    L.lost += 1
                L.req[w][k] = OPEN
            L.open.add(w)
            closed = False
            yield
        while task > 0:
            task -= 1                     # one node
            L.processed += 1
            yield
            for k in range(L.nslots):     # the request words, read once per node
                r = L.req[w][k]
                yield
                if r in (OPEN, CLOSED):
                    continue
                rcv = r - 1
                if task >= 2:             # a branch worth handing over
                    give = task // 2
                    task -= give
                    assert L.waiting[rcv] and L.mail[rcv] is None
                    L.mail[rcv] = give
                    yield
                    if plant != "no_count":   # mistake: the receiver never counted active
                        L.add_active(1)       # counted active before the wake-up
                        yield
                    L.flag[rcv] = TASK
                    yield
                else:
                    L.flag[rcv] = RETRY
                    yield
                L.req[w][k] = OPEN
                yield
        task = None
        # between subtrees the words stay open (a request may be waiting); the
        # planted mistake reopens them with a plain store, erasing such a request
        closed = plant == "erase_on_reopen"


class DidNotEnd(AssertionError):
    pass


def run(seed, nwaves, nslots, nroots, plant=None, max_steps=2_000_000):
    rng = random.Random(seed)
    roots = [rng.choice([1, 1, 2, 3, 5, 40, 200]) for _ in range(nroots)]
    L = Launch(roots, nwaves, nslots, rng)
    gens = {w: wave(L, w, plant) for w in range(nwaves)}
    steps = 0
    while gens:
        w = rng.choice(list(gens))
        try:
            next(gens[w])
        except StopIteration:
            del gens[w]
        steps += 1
        if steps >= max_steps:
            raise DidNotEnd("the launch did not end")
    return L, roots


@pytest.mark.parametrize("nslots", [1, 4])
@pytest.mark.parametrize("nwaves,nroots", [(2, 1), (3, 2), (8, 3), (16, 40), (32, 5)])
def test_protocol_loses_no_work_and_ends(nslots, nwaves, nroots):
    for seed in range(60):
        L, roots = run(seed * 7919 + nwaves * 31 + nslots, nwaves, nslots, nroots)
        assert L.processed == sum(roots), (seed, L.processed, sum(roots))
        assert L.n_active == 0 and L.min_active >= 0, (seed, L.n_active, L.min_active)
        assert L.lost == 0, seed
        assert all(m is None for m in L.mail), seed


def test_a_single_heavy_subtree_is_shared():
    """One subtree of 400 nodes and 16 waves: the others receive branches."""
    L, roots = run(3, 16, 1, 1)
    assert L.processed == 400 or L.processed == sum(roots)
    # run again with a root of a fixed size and count the waves that worked
    rng = random.Random(11)
    L = Launch([400], 16, 1, rng)
    workers = set()
    gens = {w: wave(L, w) for w in range(16)}
    while gens:
        w = rng.choice(list(gens))
        before = L.processed
        try:
            next(gens[w])
        except StopIteration:
            del gens[w]
        if L.processed > before:
            workers.add(w)
    assert L.processed == 400 and len(workers) > 4


def planted_is_caught(plant, seeds, nwaves, nroots, max_steps):
    """Runs with a planted mistake: how many break one of the invariants the
    real protocol keeps (the launch ends, no node lost or taken twice, the
    active count never below zero, a task only for a waiting wave, no request
    overwritten before its answer)."""
    caught = 0
    for seed in range(seeds):
        try:
            L, roots = run(seed, nwaves, 1, nroots, plant=plant, max_steps=max_steps)
        except AssertionError:   # the run did not end, or a task went to a wave not waiting
            caught += 1
            continue
        if L.min_active < 0 or L.n_active != 0 or L.processed != sum(roots) or L.lost:
            caught += 1
    return caught


def test_the_model_sees_a_receiver_never_counted_active():
    """A donor that wakes its receiver without counting it active lets the
    count reach zero, and the exit go out, while branches are still held."""
    assert planted_is_caught("no_count", 60, 8, 3, 500_000) > 0


def test_the_model_sees_a_refusal_consumed_with_a_plain_store():
    """Consuming a refusal with a plain store can erase the exit broadcast that
    was written over it: that wave then waits for work that never comes."""
    assert planted_is_caught("plain_retry", 200, 8, 2, 200_000) > 0


def test_the_model_sees_a_request_erased_on_reopen():
    """Reopening the request word with a plain store between two subtrees can
    erase a request that arrived meanwhile: its sender then gets no answer and
    idles until the launch ends."""
    assert planted_is_caught("erase_on_reopen", 60, 8, 40, 300_000) > 0
