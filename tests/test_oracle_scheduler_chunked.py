"""Pins for prefix caching and chunked prefill in the reference scheduler (CPU
only).

The pages: a cached prompt prefix makes that part of the prefill free, and long
prompts are split into chunks interleaved with decode ("PagedAttention: The
vLLM Paper", "Impact and Follow-Ups").  Pinned by hand-derived traces and by a
content simulation over random traces (budgets, shared prompt prefixes, both
preemption policies) in which every slot of the device and host pools is
labelled with the whole token prefix up to it, and each step's copies and
writes run in the documented order: every running request must then find its
own written tokens through its table after every step."""
import numpy as np
import pytest

from oracle.block_manager import BlockManager, BMError, EINVAL
from oracle.scheduler import Scheduler
from workloads import prefix_trace


def _steps(sc):
    out = []
    while not sc.idle():
        out.append(sc.begin_step())
        sc.end_step()
        assert len(out) < 100000
    return out


def test_chunked_prefill_worked_by_hand():
    """B=4, budget 6 tokens per step.  Step 1: request 0 (10 tokens) gets
    tokens 0-5 and uses the whole budget.  Step 2: its last 4 tokens, and
    request 1 (5 tokens) is admitted into the 2 left; request 0 produces its
    first token (slot 10).  Step 3: request 1's last 3 tokens; both produce a
    token and request 0 finishes.  Step 4: request 1's last token."""
    sc = Scheduler(BlockManager(20, 4), max_running=4, max_prefill_tokens=6)
    sc.add_request(0, 10, 2)
    sc.add_request(1, 5, 2)
    s = _steps(sc)
    assert len(s) == 4
    assert s[0]["prefill"] == [(0, 0, 6)] and s[0]["admitted"] == [(0, 10, 0)]
    assert s[0]["batch"] == [] and s[0]["slots"] == []
    assert s[1]["prefill"] == [(0, 6, 4), (1, 0, 2)] and s[1]["admitted"] == [(1, 5, 0)]
    assert s[1]["batch"] == [0] and s[1]["slots"] == [10]
    assert s[2]["prefill"] == [(1, 2, 3)] and s[2]["batch"] == [0, 1]
    assert s[2]["slots"] == [11, 17] and s[2]["finished"] == [0]
    assert s[3]["prefill"] == [] and s[3]["batch"] == [1] and s[3]["slots"] == [18]


def test_prefix_hit_within_one_step():
    """Request 1 shares request 0's first 8 tokens; both are admitted in the
    same step, and request 1 reuses the two blocks request 0 registers (the
    caller writes every chunk before any attention, so they are written by
    then): it prefills only its 9th token."""
    sc = Scheduler(BlockManager(20, 4), max_running=4)
    t0 = list(range(1, 9)) + [50, 51]
    t1 = list(range(1, 9)) + [60]
    sc.add_request(0, 10, 1, tokens=t0)
    sc.add_request(1, 9, 1, tokens=t1)
    out = sc.begin_step()
    assert out["admitted"] == [(0, 10, 0), (1, 9, 8)]
    assert out["prefill"] == [(0, 0, 10), (1, 8, 1)]
    assert sc.bm.tables[1] == [0, 1, 3] and out["slots"] == [10, 13]


def test_bad_arguments():
    with pytest.raises(BMError) as e:
        Scheduler(BlockManager(4, 4), max_running=2, max_prefill_tokens=0)
    assert e.value.code == EINVAL
    sc = Scheduler(BlockManager(4, 4), max_running=2)
    with pytest.raises(BMError):
        sc.add_request(0, 3, 1, tokens=[1, 2])


class Pools:
    """Prefix labels of the device and host pools, updated in the caller's
    order: swap-ins, swap-outs, copy-on-write, prefill chunks, token writes."""

    def __init__(self, sc):
        self.sc, self.bm = sc, sc.bm
        self.dev = [[None] * self.bm.B for _ in range(self.bm.N)]
        self.host = [[None] * self.bm.B for _ in range(max(self.bm.NH, 1))]
        self.toks = {}

    def label(self, rid, t):
        return tuple(self.toks[rid][:t + 1])

    def seq_tokens(self, r):
        known = list(r.tokens) if r.tokens is not None else [("p", r.rid, i) for i in range(r.prompt)]
        return known + [("g", r.rid, i) for i in range(r.generated + 1)]

    def slot(self, rid, t):
        tab = self.bm.tables[rid]
        return tab[t // self.bm.B], t % self.bm.B

    def step(self, out):
        reqs = {r.rid: r for r in list(self.sc.running) + list(self.sc.swapped) +
                list(self.sc.waiting)}
        for rid, r in reqs.items():
            self.toks[rid] = self.seq_tokens(r)
        for h, d in out["swap_in"]:
            self.dev[d] = list(self.host[h])
        for d, h in out["swap_out"]:
            self.host[h] = list(self.dev[d])
        for src, dst in out["cow"]:
            self.dev[dst] = list(self.dev[src])
        for rid, start, n in out["prefill"]:
            for t in range(start, start + n):
                b, o = self.slot(rid, t)
                self.dev[b][o] = self.label(rid, t)
        B = self.bm.B
        for rid, slot in zip(out["batch"], out["slots"]):
            t = self.bm.lens[rid] - 1
            assert self.slot(rid, t) == (slot // B, slot % B)
            self.dev[slot // B][slot % B] = self.label(rid, t)

    def check(self):
        B = self.bm.B
        for r in self.sc.running:
            written = r.prefilled if r.prefilled < r.target else self.bm.lens[r.rid]
            for t in range(written):
                b, o = self.slot(r.rid, t)
                assert self.dev[b][o] == self.label(r.rid, t), ("device", r.rid, t)
        for r in self.sc.swapped:
            written = r.prefilled if r.prefilled < r.target else self.bm.lens[r.rid]
            table = self.bm.host_tables[r.rid]
            for t in range(written):
                assert self.host[table[t // B]][t % B] == self.label(r.rid, t), ("host", r.rid, t)


def chunked_trace_run(seed, sched_cls=Scheduler):
    rng = np.random.default_rng(6100 + seed)
    B = int(rng.choice([2, 4, 16]))
    trace = prefix_trace(rng, int(rng.integers(5, 30)), prefix_median=3 * B,
                         suffix_median=B, out_median=8, max_prefix=8 * B, max_suffix=4 * B,
                         max_out=30, vocab=5)
    N = max(-(-(p + m) // B) for _, p, m, _ in trace) + int(rng.integers(0, 20))
    swap = bool(rng.random() < 0.5)
    budget = [None, int(rng.integers(1, 4 * B))][int(rng.random() < 0.7)]
    bm = BlockManager(N, B, rng.permutation(N))
    if swap:
        bm.set_host_pool(int(rng.integers(1, 3 * N)))
    sc = sched_cls(bm, int(rng.integers(1, 10)), swap=swap, max_prefill_tokens=budget)
    for rid, p, m, toks in trace:
        sc.add_request(rid, p, m, tokens=toks if rng.random() < 0.9 else None)
    pools = Pools(sc)
    want = {rid: m for rid, _, m, _ in trace}
    produced = {rid: 0 for rid in want}
    hits = steps = 0
    while not sc.idle():
        out = sc.begin_step()
        steps += 1
        assert steps < 100000
        pools.step(out)
        pools.check()
        if budget is not None:
            assert sum(n for _, _, n in out["prefill"]) <= budget
        for rid in out["batch"]:
            produced[rid] += 1
        hits += sum(c for _, _, c in out["admitted"])
        sc.end_step()
    assert produced == want
    assert bm.num_free() == N
    return hits


@pytest.mark.parametrize("seed", range(30))
def test_chunked_and_cached_traces_keep_every_request_content(seed):
    chunked_trace_run(seed)


def test_traces_hit_the_prefix_cache():
    assert sum(chunked_trace_run(s) > 0 for s in range(30)) >= 20
