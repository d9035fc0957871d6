"""The C++ continuous-batching scheduler (through the C ABI) against the
reference scheduler: identical steps (batch, slots, copy pairs, admissions with
their contexts, preemptions, finishes, swap pairs), identical accounting and
identical block-manager state after every step, under all three policies
(CPU only)."""
import ctypes

import numpy as np
import pytest

from oracle.block_manager import BlockManager as RefBM
from oracle.scheduler import Scheduler as RefSched
from workloads import request_trace


def run_parity(pkv, seed, policy):
    reserve, swap = policy == "reserve", policy == "swap"
    rng = np.random.default_rng(1500 + seed)
    B = int(rng.choice([1, 4, 16, 32]))
    trace = request_trace(rng, int(rng.integers(1, 60)), prompt_median=50, out_median=30,
                          max_prompt=200, max_out=80)
    N = max(-(-(p + m) // B) for _, p, m in trace) + int(rng.integers(0, 60))
    order = rng.permutation(N)
    max_running = int(rng.integers(1, 16))
    nbm, rbm = pkv.BlockManager(N, B, order), RefBM(N, B, order)
    if swap:
        NH = int(rng.integers(1, 2 * N))
        nbm.set_host_pool(NH)
        rbm.set_host_pool(NH)
    nat = pkv.Scheduler(nbm, max_running, reserve, swap)
    ref = RefSched(rbm, max_running, reserve, swap)
    for rid, p, m in trace:
        nat.add_request(rid, p, m)
        ref.add_request(rid, p, m)
    steps = swaps = 0
    while not ref.idle():
        a, b = nat.begin_step(), ref.begin_step()
        assert a == {k: (list(v) if k != "admitted" else [tuple(x) for x in v])
                     for k, v in b.items()}
        held, committed, nw, nr, ns = nat.stats()
        assert (held, committed) == (ref.tokens_held(), ref.slots_committed())
        assert (nw, nr, ns) == (len(ref.waiting), len(ref.running), len(ref.swapped))
        ids = a["batch"]
        if ids:
            maxb = max(len(rbm.tables[i]) for i in ids)
            t, l = nbm.fill_batch(ids, maxb)
            rt, rl = rbm.fill_batch(ids, maxb)
            assert t.tolist() == rt and l.tolist() == rl
        nat.end_step()
        ref.end_step()
        refc, free = nbm.snapshot()
        assert refc == rbm.ref and free == list(rbm.free)
        if swap:
            assert nbm.host_free_queue() == list(rbm.host_free)
            swaps += len(a["swapped_out"])
        steps += 1
    assert nat.stats() == (0, 0, 0, 0, 0)
    assert steps > 0
    return swaps


@pytest.mark.parametrize("policy", ["paged", "reserve", "swap"])
@pytest.mark.parametrize("seed", range(10))
def test_random_traces_bit_exact(pkv, seed, policy):
    run_parity(pkv, seed, policy)


def test_swap_parity_traces_do_swap(pkv):
    assert sum(run_parity(pkv, s, "swap") > 0 for s in range(10)) >= 5


def test_policy_word_is_validated(pkv):
    bm = pkv.BlockManager(4, 16)
    h = ctypes.c_void_p()
    for bad in (pkv.PKV_SCHED_RESERVE_MAX | pkv.PKV_SCHED_SWAP, 4, -1):
        assert pkv.lib.pkv_sched_create(bm._h, 2, bad, 0, ctypes.byref(h)) == pkv.PKV_EINVAL
    assert pkv.lib.pkv_sched_create(bm._h, 2, 0, -1, ctypes.byref(h)) == pkv.PKV_EINVAL


def test_native_error_paths(pkv):
    bm = pkv.BlockManager(4, 16)
    sc = pkv.Scheduler(bm, 2)
    sc.add_request(0, 10, 5)
    with pytest.raises(pkv.PkvError) as e:
        sc.add_request(0, 10, 5)
    assert e.value.code == pkv.PKV_EEXIST
    for bad in ((1, -1, 5), (2, 10, 0), (3, 60, 10)):
        with pytest.raises(pkv.PkvError) as e:
            sc.add_request(*bad)
        assert e.value.code == pkv.PKV_EINVAL
    with pytest.raises(pkv.PkvError):
        sc.end_step()
    sc.begin_step()
    with pytest.raises(pkv.PkvError):
        sc.begin_step()
    sc.end_step()
    with pytest.raises(pkv.PkvError):
        pkv.Scheduler(bm, 0)
    assert bm.geometry() == (4, 16)


@pytest.mark.parametrize("seed", range(24))
def test_chunked_cached_traces_bit_exact(pkv, seed):
    """Prefill budgets, prompt token ids with shared prefixes, and both
    preemption policies: identical steps (prefill chunks and cached counts
    included), accounting, block-manager state and prefix-cache size."""
    from workloads import prefix_trace
    rng = np.random.default_rng(6600 + seed)
    B = int(rng.choice([2, 4, 16]))
    trace = prefix_trace(rng, int(rng.integers(5, 40)), prefix_median=3 * B, suffix_median=B,
                         out_median=8, max_prefix=8 * B, max_suffix=4 * B, max_out=30, vocab=5)
    N = max(-(-(p + m) // B) for _, p, m, _ in trace) + int(rng.integers(0, 20))
    swap = bool(rng.random() < 0.5)
    budget = [None, int(rng.integers(1, 4 * B))][int(rng.random() < 0.7)]
    max_running = int(rng.integers(1, 10))
    order = rng.permutation(N)
    nbm, rbm = pkv.BlockManager(N, B, order), RefBM(N, B, order)
    if swap:
        NH = int(rng.integers(1, 3 * N))
        nbm.set_host_pool(NH)
        rbm.set_host_pool(NH)
    nat = pkv.Scheduler(nbm, max_running, False, swap, budget)
    ref = RefSched(rbm, max_running, False, swap, budget)
    for rid, p, m, toks in trace:
        use = rng.random() < 0.9
        nat.add_request(rid, p, m, tokens=toks if use else None)
        ref.add_request(rid, p, m, tokens=toks if use else None)
    steps = 0
    while not ref.idle():
        a, b = nat.begin_step(), ref.begin_step()
        assert a == {k: [tuple(x) if isinstance(x, tuple) else x for x in v] for k, v in b.items()}
        held, committed, nw, nr, ns = nat.stats()
        assert (held, committed) == (ref.tokens_held(), ref.slots_committed())
        assert (nw, nr, ns) == (len(ref.waiting), len(ref.running), len(ref.swapped))
        nat.end_step()
        ref.end_step()
        refc, free = nbm.snapshot()
        assert refc == rbm.ref and free == list(rbm.free)
        assert nbm.cached_blocks() == rbm.cached_blocks()
        steps += 1
    assert nat.stats() == (0, 0, 0, 0, 0)
