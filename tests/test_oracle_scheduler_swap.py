"""Pins for the swap policy of the reference scheduler (CPU only).

The pages: under memory pressure a request is preempted by moving its KV blocks
to CPU memory, or by dropping them for later recomputation ("PagedAttention:
The vLLM Paper", "Implementation Essentials"; "The Core Idea", analogy table,
"Swapping").  Pinned here: a hand-derived trace, the case where the victim has
no KV yet, and a content simulation over random traces in which every slot of
the device and host pools holds a (request, position) label and each step's
copies and writes run in the documented order -- so every running request
must find its own tokens on the device after every step, and every swapped
one on the host."""
import numpy as np
import pytest

from oracle.block_manager import BlockManager, BMError, EINVAL
from oracle.scheduler import Scheduler
from workloads import request_trace


def _bm(N, B, NH):
    bm = BlockManager(N, B)
    bm.set_host_pool(NH)
    return bm


def _run(sc):
    steps = []
    while not sc.idle():
        steps.append(sc.begin_step())
        sc.end_step()
        assert len(steps) < 100000
    return steps


def test_swap_trace_worked_by_hand():
    """B=4, 6 device blocks, 8 host blocks; two requests of 8 + 9 tokens.
    Step 1 admits both (blocks [0,1] and [2,3]) and appends into 4 and 5.
    Step 5: request 0 needs a fifth block, none is free, so the younger
    request 1 (blocks [2,3,5], 12 tokens) goes to host blocks 0,1,2 and request
    0 takes block 2.  Request 1 cannot come back (3 blocks, 2 free) until
    request 0 finishes in step 9 and frees [0,1,4,2,3]; step 10 brings it back
    into blocks 5,0,1 and it appends into 4.  It is never recomputed."""
    sc = Scheduler(_bm(6, 4, 8), max_running=4, swap=True)
    sc.add_request(0, 8, 9)
    sc.add_request(1, 8, 9)
    steps = _run(sc)
    assert len(steps) == 14
    assert steps[0]["admitted"] == [(0, 8, 0), (1, 8, 0)] and steps[0]["slots"] == [16, 20]
    assert all(not s["admitted"] for s in steps[1:])             # no recomputation
    assert all(not s["preempted"] for s in steps)
    s5 = steps[4]
    assert s5["swap_out"] == [(2, 0), (3, 1), (5, 2)] and s5["swapped_out"] == [1]
    assert s5["batch"] == [0] and s5["slots"] == [8]
    for s in steps[5:9]:                                          # steps 6-9: no room
        assert s["swap_in"] == [] and s["batch"] == [0]
    assert steps[8]["finished"] == [0]
    s10 = steps[9]
    assert s10["swap_in"] == [(0, 5), (1, 0), (2, 1)] and s10["swapped_in"] == [1]
    assert s10["batch"] == [1] and s10["slots"] == [16]
    assert steps[13]["finished"] == [1] and steps[13]["slots"] == [8]
    assert sc.bm.num_free() == 6 and sc.bm.num_free_host() == 8


def test_a_victim_without_kv_is_dropped_not_swapped():
    """B=4, 4 device blocks: request 0 takes [0,1], request 1 takes [2], and
    request 0's append takes the last block, so request 1's append finds none.
    Request 1 was admitted in this step and its prefill is not written yet:
    it is dropped although the host has room."""
    sc = Scheduler(_bm(4, 4, 8), max_running=2, swap=True)
    sc.add_request(0, 8, 5)
    sc.add_request(1, 4, 3)
    out = sc.begin_step()
    assert out["preempted"] == [1] and out["swap_out"] == []
    assert out["admitted"] == [(0, 8, 0)] and out["batch"] == [0]


def test_swap_and_reserve_do_not_combine():
    with pytest.raises(BMError) as e:
        Scheduler(_bm(4, 4, 4), max_running=2, reserve_max=True, swap=True)
    assert e.value.code == EINVAL


class Pools:
    """Labels of the device and host pools, updated step by step in the order
    the caller must run a step: swap-ins, swap-outs, copy-on-write copies,
    prefill writes, then each running request's new token."""

    def __init__(self, bm):
        self.bm = bm
        self.dev = [[None] * bm.B for _ in range(bm.N)]
        self.host = [[None] * bm.B for _ in range(bm.NH)]

    def _slot(self, rid, t):
        b = self.bm.tables[rid][t // self.bm.B]
        return b, t % self.bm.B

    def step(self, out):
        for h, d in out["swap_in"]:
            self.dev[d] = list(self.host[h])
        for d, h in out["swap_out"]:
            self.host[h] = list(self.dev[d])
        for src, dst in out["cow"]:
            self.dev[dst] = list(self.dev[src])
        for rid, start, n in out["prefill"]:
            for t in range(start, start + n):
                b, o = self._slot(rid, t)
                self.dev[b][o] = (rid, t)
        B = self.bm.B
        for rid, slot in zip(out["batch"], out["slots"]):
            t = self.bm.lens[rid] - 1
            assert self._slot(rid, t) == (slot // B, slot % B)
            self.dev[slot // B][slot % B] = (rid, t)

    def check(self, running, swapped):
        B = self.bm.B
        for rid in running:
            for t in range(self.bm.lens[rid]):
                b, o = self._slot(rid, t)
                assert self.dev[b][o] == (rid, t), ("device", rid, t)
        for rid in swapped:
            table = self.bm.host_tables[rid]
            for t in range(self.bm.lens[rid]):
                assert self.host[table[t // B]][t % B] == (rid, t), ("host", rid, t)


def swap_trace_run(seed, sched_cls=Scheduler):
    rng = np.random.default_rng(3100 + seed)
    B = int(rng.choice([2, 4, 16]))
    trace = request_trace(rng, int(rng.integers(5, 40)), prompt_median=30, out_median=25,
                          max_prompt=100, max_out=80)
    N = max(-(-(p + m) // B) for _, p, m in trace) + int(rng.integers(0, 30))
    NH = int(rng.integers(1, 3 * N))
    max_running = int(rng.integers(1, 12))
    bm = _bm(N, B, NH)
    sc = sched_cls(bm, max_running, swap=True)
    for rid, p, m in trace:
        sc.add_request(rid, p, m)
    pools = Pools(bm)
    want = {rid: m for rid, _, m in trace}
    produced = {rid: 0 for rid in want}
    admitted_order, swaps = [], 0
    steps = 0
    while not sc.idle():
        out = sc.begin_step()
        steps += 1
        assert steps < 100000
        pools.step(out)
        swapped_now = [r.rid for r in sc.swapped]
        pools.check(out["batch"], swapped_now)
        # a request waits for admission while any preempted one is still out
        if out["admitted"]:
            assert set(swapped_now) <= set(out["swapped_out"])
        # victims are the youngest: swapped-out and dropped ones are the tail
        assert 0 < len(out["batch"]) <= max_running
        for rid in out["batch"]:
            produced[rid] += 1
        admitted_order += [a[0] for a in out["admitted"]]
        swaps += len(out["swapped_out"])
        # a swapped request resumes with the tokens it held
        for rid in out["swapped_in"]:
            assert rid in out["batch"] or rid in out["swapped_out"] or rid in out["preempted"]
        sc.end_step()
    assert produced == want
    firsts = list(dict.fromkeys(admitted_order))
    assert firsts == sorted(firsts)
    assert bm.num_free() == N and bm.num_free_host() == NH
    return swaps


@pytest.mark.parametrize("seed", range(24))
def test_swap_invariants_on_random_traces(seed):
    swap_trace_run(seed)


def test_random_traces_do_swap():
    assert sum(swap_trace_run(s) > 0 for s in range(24)) >= 12
