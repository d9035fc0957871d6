"""pkv_pack_step (host only): the packed step metadata equals what the block
manager and the plan builder give one call at a time -- chunk slots and
tables, decode tables, lengths and plan, the K/V row list, the block copy
pairs -- on scheduler traces with chunked prefill, preemption by drop and by
swap, and prefix-cache hits.  Each array starts on a 16-byte boundary."""
import numpy as np
import pytest

import workloads as W


def expected(bm, pkv, st, max_blocks, Hkv, P, B):
    ids, chunks = st["batch"], st["prefill"]
    exp = {"n_prefill_rows": sum(c for _, _, c in chunks)}
    if chunks:
        exp["slots"] = np.concatenate([bm.slots(r, a, c)[:c] for r, a, c in chunks])
        pf_lens = np.array([a + c for _, a, c in chunks], np.int32)
        width = max(1, -(-int(pf_lens.max()) // B))
        t, _ = bm.fill_batch([r for r, _, _ in chunks], max_blocks)
        exp["pf_tables"] = t[:, :width]
        exp["pf_lens"] = pf_lens
        exp["pf_start"] = np.concatenate([[0], np.cumsum([c for _, _, c in chunks])])
        exp["pf_max_rows"] = max(c for _, _, c in chunks)
    pairs = [np.stack([np.full(c, r), np.arange(a, a + c)], 1) for r, a, c in chunks]
    if ids:
        tables, lens = bm.fill_batch(ids, max_blocks)
        mcl = int(lens.max())
        width = max(1, -(-mcl // B))
        exp["tables"] = tables[:, :width]
        exp["lens"] = lens
        exp["plan"] = pkv.attention_plan(lens, Hkv, B, width, mcl, P)
        pairs.append(np.stack([np.asarray(ids), lens.astype(np.int64) - 1], 1))
    exp["pairs"] = np.concatenate(pairs).astype(np.int64) if pairs else np.zeros((0, 2), np.int64)
    return exp


@pytest.mark.parametrize("seed,swap,budget", [(0, False, None), (1, True, None),
                                              (2, False, 96), (3, True, 64), (4, True, None)])
def test_pack_step_matches_one_call_at_a_time(pkv, seed, swap, budget):
    rng = np.random.default_rng(1200 + seed)
    B, Hkv, P = 16, 4, int(rng.choice([64, 128, 512]))
    N = 40
    bm = pkv.BlockManager(N, B, rng.permutation(N).astype(np.int32))
    if swap:
        bm.set_host_pool(24)
    trace = W.request_trace(rng, 40, prompt_median=40, out_median=30, max_prompt=300,
                            max_out=120)
    max_blocks = -(-max(p + m for _, p, m in trace) // B)
    sched = pkv.Scheduler(bm, 16, swap=swap, max_prefill_tokens=budget)
    shared = [rng.integers(0, 1000, 64) for _ in range(3)]   # prompt prefixes some requests share
    for rid, p_, m_ in trace:
        tokens = None
        if rid % 2 and p_ > 64:
            tokens = np.concatenate([shared[rid % 3], rng.integers(0, 1000, p_ - 64)])
        sched.add_request(rid, p_, m_, tokens=tokens)
    buf = np.zeros(8, np.int32)
    seen = {"cow": 0, "swap": 0, "preempt": 0, "grow": 0}
    for _ in range(5000):
        st = sched.begin_step()
        lay = pkv.StepPack()
        while not sched.pack_step(max_blocks, Hkv, P, buf, lay):
            assert lay.total_words > buf.shape[0]
            buf = np.zeros(lay.total_words, np.int32)
            seen["grow"] += 1
        offs = [lay.slots_off, lay.pf_tables_off, lay.pf_lens_off, lay.pf_start_off,
                lay.tables_off, lay.lens_off, lay.plan_off, lay.pairs_off, lay.swap_in_off,
                lay.swap_out_off, lay.cow_off]
        assert all(o % 4 == 0 for o in offs) and lay.total_words <= buf.shape[0]
        exp = expected(bm, pkv, st, max_blocks, Hkv, P, B)
        n, nc, rows = len(st["batch"]), len(st["prefill"]), exp["n_prefill_rows"]
        assert lay.n_prefill_rows == rows
        if nc:
            got = buf[lay.slots_off:lay.slots_off + 2 * rows].view(np.int64)
            assert np.array_equal(got, exp["slots"])
            w = lay.pf_width
            assert np.array_equal(buf[lay.pf_tables_off:lay.pf_tables_off + nc * w]
                                  .reshape(nc, w), exp["pf_tables"])
            assert np.array_equal(buf[lay.pf_lens_off:lay.pf_lens_off + nc], exp["pf_lens"])
            assert np.array_equal(buf[lay.pf_start_off:lay.pf_start_off + nc + 1],
                                  exp["pf_start"])
            assert lay.pf_max_rows == exp["pf_max_rows"]
        if n:
            w = lay.width
            assert np.array_equal(buf[lay.tables_off:lay.tables_off + n * w].reshape(n, w),
                                  exp["tables"])
            assert np.array_equal(buf[lay.lens_off:lay.lens_off + n], exp["lens"])
            assert lay.max_context == int(exp["lens"].max())
            words, ni, nm = exp["plan"]
            assert (lay.n_items, lay.n_merge) == (ni, nm)
            assert np.array_equal(buf[lay.plan_off:lay.plan_off + 4 * ni + nm], words)
        pairs = buf[lay.pairs_off:lay.pairs_off + 4 * (rows + n)].view(np.int64).reshape(-1, 2)
        assert np.array_equal(pairs, exp["pairs"])
        for key, off in (("swap_in", lay.swap_in_off), ("swap_out", lay.swap_out_off),
                         ("cow", lay.cow_off)):
            k = len(st[key])
            got = buf[off:off + 2 * k].reshape(-1, 2).tolist()
            assert [tuple(x) for x in got] == list(st[key])
        seen["cow"] += len(st["cow"])
        seen["swap"] += len(st["swap_out"]) + len(st["swap_in"])
        seen["preempt"] += len(st["preempted"])
        sched.end_step()
        _, _, nw, nr, ns = sched.stats()
        if nw == 0 and nr == 0 and ns == 0:
            break
    else:
        pytest.fail("trace did not finish")
    assert seen["grow"] >= 1
    assert seen["preempt"] + seen["swap"] > 0    # the pool is small enough to preempt
