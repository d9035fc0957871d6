"""The C++ continuous-batching scheduler (through the C ABI) against the
reference scheduler: identical steps (batch, slots, copy pairs, admissions with
their contexts, preemptions, finishes), identical accounting and identical
block-manager state after every step, under both policies (CPU only)."""
import numpy as np
import pytest

from oracle.block_manager import BlockManager as RefBM
from oracle.scheduler import Scheduler as RefSched
from workloads import request_trace


@pytest.mark.parametrize("reserve", [False, True])
@pytest.mark.parametrize("seed", range(10))
def test_random_traces_bit_exact(pkv, seed, reserve):
    rng = np.random.default_rng(1500 + seed)
    B = int(rng.choice([1, 4, 16, 32]))
    trace = request_trace(rng, int(rng.integers(1, 60)), prompt_median=50, out_median=30,
                          max_prompt=200, max_out=80)
    N = max(-(-(p + m) // B) for _, p, m in trace) + int(rng.integers(0, 60))
    order = rng.permutation(N)
    max_running = int(rng.integers(1, 16))
    nbm, rbm = pkv.BlockManager(N, B, order), RefBM(N, B, order)
    nat = pkv.Scheduler(nbm, max_running, reserve)
    ref = RefSched(rbm, max_running, reserve)
    for rid, p, m in trace:
        nat.add_request(rid, p, m)
        ref.add_request(rid, p, m)
    steps = 0
    while not ref.idle():
        a, b = nat.begin_step(), ref.begin_step()
        assert a == {k: (list(v) if k != "admitted" else [tuple(x) for x in v])
                     for k, v in b.items()}
        held, committed, nw, nr = nat.stats()
        assert (held, committed) == (ref.tokens_held(), ref.slots_committed())
        assert (nw, nr) == (len(ref.waiting), len(ref.running))
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
        steps += 1
    assert nat.stats() == (0, 0, 0, 0)
    assert steps > 0


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
