"""Pins for the reference continuous-batching scheduler (CPU only): the pages'
iteration-level figure, and invariants that hold after every step of many
seeded traces under both policies."""
import json
import os

import numpy as np
import pytest

from oracle.block_manager import BlockManager, BMError, EEXIST, EINVAL
from oracle.scheduler import Scheduler
from workloads import request_trace

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_iteration_level_figure():
    with open(os.path.join(GOLDEN, "continuous_batching_figure.json")) as f:
        g = json.load(f)
    names = ["A", "B", "C", "D"]
    new_tokens = {"A": 2, "B": 6, "C": 6, "D": 3}
    sc = Scheduler(BlockManager(64, 16), max_running=3)
    for i, n in enumerate(names):
        sc.add_request(i, 20, new_tokens[n])
    steps = []
    while not sc.idle():
        out = sc.begin_step()
        steps.append(out)
        sc.end_step()
    label = lambda ids: [names[i] for i in ids]
    a_done = next(k for k, o in enumerate(steps) if names.index(g["finishes"]) in o["finished"])
    assert label(steps[a_done]["batch"]) == g["batch_before"]
    # the very next iteration: A has left and D has joined
    nxt = steps[a_done + 1]
    assert label(nxt["batch"]) == g["batch_after"]
    assert label([a[0] for a in nxt["admitted"]]) == [g["joins"]]
    # D waited only because of the batch limit, not for B and C to finish
    b_done = next(k for k, o in enumerate(steps) if 1 in o["finished"])
    assert a_done + 1 < b_done


def test_admission_needs_free_blocks_not_a_contiguous_region():
    """The pool's free blocks are scattered (3 and 5 of 8, as in the block-pool
    figure); a two-block request is admitted into them."""
    bm = BlockManager(8, 16)
    for sid in (10, 11, 10, 12, 11, 12, 10, 11):     # A, B, A, C, B, C, A, B
        if sid in bm.tables:
            for _ in range(16):
                bm.append_slot(sid)
        else:
            bm.add_seq(sid, 16)
    bm.free_seq(12)
    assert sorted(bm.free) == [3, 5]
    sc = Scheduler(bm, max_running=4)
    sc.add_request(0, 31, 1)        # 32 tokens after its step: exactly 2 blocks
    out = sc.begin_step()
    assert out["admitted"] == [(0, 31, 0)] and bm.tables[0] == [3, 5]


def test_reserve_policy_holds_the_maximum_length():
    """The max-length reservation of the earlier systems: a request is admitted
    only when its whole maximum length is free, and its committed slots are
    that maximum, whatever it holds so far."""
    B = 16
    sc = Scheduler(BlockManager(10, B), max_running=8, reserve_max=True)
    sc.add_request(0, 100, 60)      # ceil(160/16) = 10 blocks: the whole pool
    sc.add_request(1, 1, 1)         # 1 block: must wait although 3 blocks are free
    out = sc.begin_step()
    assert out["batch"] == [0] and sc.slots_committed() == 10 * B
    assert sc.tokens_held() == 101
    assert sc.bm.num_free() == 10 - 7
    sc.end_step()
    paged = Scheduler(BlockManager(10, B), max_running=8)
    paged.add_request(0, 100, 60)
    paged.add_request(1, 1, 1)
    assert paged.begin_step()["batch"] == [0, 1]


def run_trace(sc, trace):
    for rid, p, m in trace:
        sc.add_request(rid, p, m)
    steps = []
    while not sc.idle():
        out = sc.begin_step()
        steps.append((out, sc.tokens_held(), sc.slots_committed(), sc.bm.num_free()))
        sc.end_step()
        assert len(steps) < 100000
    return steps


@pytest.mark.parametrize("reserve", [False, True])
@pytest.mark.parametrize("seed", range(6))
def test_invariants_on_random_traces(seed, reserve):
    rng = np.random.default_rng(1200 + seed)
    B = int(rng.choice([4, 16]))
    trace = request_trace(rng, int(rng.integers(5, 40)), prompt_median=40, out_median=20,
                          max_prompt=120, max_out=60)
    N = max(-(-(p + m) // B) for _, p, m in trace) + int(rng.integers(0, 40))
    max_running = int(rng.integers(1, 12))
    sc = Scheduler(BlockManager(N, B), max_running, reserve_max=reserve)
    steps = run_trace(sc, trace)
    want = {rid: m for rid, _, m in trace}
    produced = {rid: 0 for rid in want}
    admitted_order, finished = [], []
    for out, held, committed, nfree in steps:
        assert 0 < len(out["batch"]) <= max_running
        for rid in out["batch"]:
            produced[rid] += 1
        admitted_order += [a[0] for a in out["admitted"]]
        finished += out["finished"]
        assert held <= committed
        if reserve:
            assert not out["preempted"]
        else:
            # only a sequence's last block may be partly empty
            assert committed - held <= (B - 1) * len(out["batch"])
            assert committed == (N - nfree) * B
        if out["preempted"]:
            assert not reserve
    # every request produced exactly its tokens and finished once
    assert produced == want
    assert sorted(finished) == sorted(want)
    # first-come first-served: first admissions follow submission order
    firsts = list(dict.fromkeys(admitted_order))
    assert firsts == sorted(firsts)
    # everything returned to the pool
    assert sc.bm.num_free() == N and sc.reserved == 0


def test_preemption_drops_the_youngest_and_recomputes_it():
    B = 4
    sc = Scheduler(BlockManager(6, B), max_running=4)
    sc.add_request(0, 8, 9)   # 2 blocks, grows to 17 tokens: 5 blocks
    sc.add_request(1, 8, 9)
    out = sc.begin_step()     # both admitted: 2 + 2 blocks, then 1 + 1 for the appends
    assert out["batch"] == [0, 1] and sc.bm.num_free() == 0
    sc.end_step()
    seen = []
    while not sc.idle():
        out = sc.begin_step()
        seen.append(out)
        sc.end_step()
    pre = [k for k, o in enumerate(seen) if o["preempted"]]
    assert pre and seen[pre[0]]["preempted"] == [1]          # the younger request
    back = next(o for o in seen[pre[0]:] if o["admitted"])
    rid, ctx, _ = back["admitted"][0]
    assert rid == 1 and ctx > 8                                # prompt + kept tokens


def test_error_paths():
    sc = Scheduler(BlockManager(4, 16), max_running=2)
    sc.add_request(0, 10, 5)
    with pytest.raises(BMError) as e:
        sc.add_request(0, 10, 5)
    assert e.value.code == EEXIST
    for bad in ((1, -1, 5), (2, 10, 0), (3, 60, 10)):     # 70 tokens > 4 blocks of 16
        with pytest.raises(BMError) as e:
            sc.add_request(*bad)
        assert e.value.code == EINVAL
    with pytest.raises(BMError):
        sc.end_step()                                      # no step in progress
    sc.begin_step()
    with pytest.raises(BMError):
        sc.begin_step()                                    # end_step() is due
    sc.end_step()
    with pytest.raises(BMError):
        Scheduler(BlockManager(4, 16), max_running=0)
