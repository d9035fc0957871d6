"""Pins of the reference block manager's truncate (speculative drafts): a
hand-worked example, the block-manager invariants on random scripts that mix
truncations with everything else, and a content simulation in which every slot
carries the token prefix whose KV it holds -- speculative steps that append
drafts and keep a random number of them, rollbacks into prompt blocks that the
prefix cache holds, copy-on-write and prefix-cache hits -- so every live
sequence must find its own tokens' KV at every position (CPU only)."""
import numpy as np
import pytest

from oracle.block_manager import OK, BlockManager, BMError, run_ops
from tests.test_oracle_block_manager import check_invariants
from workloads import random_script


def test_truncate_worked_example():
    # B = 4, ascending pool of 8: 10 tokens hold blocks 0, 1, 2 (2 of 4 slots in 2)
    bm = BlockManager(8, 4)
    bm.add_seq(7, 10)
    assert bm.block_table(7) == [0, 1, 2]
    bm.truncate(7, 5)                     # keep ceil(5/4) = 2 blocks; block 2 goes back
    assert bm.block_table(7) == [0, 1] and bm.lens[7] == 5
    assert list(bm.free) == [3, 4, 5, 6, 7, 2]
    slot, src, dst = bm.append_slot(7)    # position 5: block 1, offset 1, in place
    assert (slot, src, dst) == (1 * 4 + 1, -1, -1)
    bm.truncate(7, 4)                     # a block boundary: block 1 goes back too
    assert bm.block_table(7) == [0] and list(bm.free) == [3, 4, 5, 6, 7, 2, 1]
    assert bm.append_slot(7) == (3 * 4, -1, -1)   # position 4 opens a new block: 3
    bm.truncate(7, 5)                     # the sequence's own length: no change
    assert bm.block_table(7) == [0, 3] and bm.lens[7] == 5
    bm.truncate(7, 0)                     # everything back, blocks in logical order
    assert bm.block_table(7) == [] and list(bm.free) == [4, 5, 6, 7, 2, 1, 0, 3]
    # a shared block loses one reference only
    bm.add_seq(1, 6)                      # blocks 4, 5
    bm.fork(1, 2)
    bm.truncate(2, 3)
    assert bm.block_table(2) == [4] and bm.ref[4] == 2 and bm.ref[5] == 1
    assert bm.append_slot(2) == (6 * 4 + 3, 4, 6)   # writes into shared block 4: copy
    for bad in (-1, 5):
        with pytest.raises(BMError):
            bm.truncate(2, bad)
    with pytest.raises(BMError):
        bm.truncate(99, 0)


@pytest.mark.parametrize("seed", range(30))
def test_invariants_with_truncation(seed):
    rng = np.random.default_rng(1500 + seed)
    N, B = int(rng.integers(4, 40)), int(rng.choice([1, 2, 4, 16]))
    bm = BlockManager(N, B, rng.permutation(N))
    seen = 0
    for op in random_script(rng, 300, max_seqs=6, max_add=5 * B, truncate=True):
        before = (bm.snapshot(), {k: list(v) for k, v in bm.tables.items()}, dict(bm.lens))
        codes, _ = run_ops(bm, [op])
        if codes[0] != OK:      # every failing call leaves the state unchanged
            assert (bm.snapshot(), bm.tables, bm.lens) == before
        elif op[0] == "truncate_by":
            seen += 1
            sid, L0 = op[1], before[2][op[1]]
            assert bm.lens[sid] == L0 - op[2]
            assert bm.tables[sid] == before[1][sid][:-(-(L0 - op[2]) // B)]
        check_invariants(bm)
    assert seen > 3
    for sid in list(bm.tables):
        bm.free_seq(sid)
    assert bm.num_free() == N and all(r == 0 for r in bm.ref)


def simulate_speculative(seed, bm_cls=BlockManager, steps=250, log=None):
    """Content simulation; returns the number of prefix-cache hits seen.  `log`
    (a list) receives every block-manager call made, in order, for replay."""
    rng = np.random.default_rng(seed)
    B = int(rng.choice([2, 4]))
    N = 40
    bm = bm_cls(N, B, rng.permutation(N))
    content = {}            # slot -> the token prefix whose KV the slot holds
    toks = {}               # live sequence -> its token ids
    prompts = [[int(x) for x in rng.integers(0, 4, 12)] for _ in range(3)]
    live, next_sid, hits = [], 0, 0

    def rec(*op):
        if log is not None:
            log.append(op)

    def append(sid, tok):
        rec("append", sid)
        slot, src, dst = bm.append_slot(sid)
        if src >= 0:        # copy-on-write: the device copies the whole block
            for o in range(B):
                if src * B + o in content:
                    content[dst * B + o] = content[src * B + o]
        toks[sid].append(tok)
        content[slot] = tuple(toks[sid])

    for _ in range(steps):
        r = rng.random()
        if r < 0.15 or not live:
            pr = prompts[int(rng.integers(3))] + [int(x) for x in rng.integers(0, 4, int(rng.integers(1, 6)))]
            sid = next_sid
            next_sid += 1
            rec("add_prefix", sid, list(pr), len(pr))
            try:
                cached = bm.add_seq_prefix(sid, pr, len(pr))
            except BMError:
                continue
            hits += cached
            toks[sid] = list(pr)
            t = bm.tables[sid]
            for p in range(cached, len(pr)):      # the prefill writes the rest
                content[t[p // B] * B + p % B] = tuple(pr[:p + 1])
            rec("register", sid, list(pr), len(pr))
            bm.register_prefix(sid, pr, len(pr))
            live.append(sid)
        elif r < 0.25:
            sid = live.pop(int(rng.integers(len(live))))
            rec("free", sid)
            bm.free_seq(sid)
            del toks[sid]
        elif r < 0.35:
            # roll back anywhere, even into the cached prompt blocks, then go on
            sid = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, bm.lens[sid] + 1))
            rec("truncate", sid, n)
            bm.truncate(sid, n)
            del toks[sid][n:]
            try:
                for _ in range(int(rng.integers(1, 4))):
                    append(sid, int(rng.integers(0, 4)))
            except BMError:
                pass
        else:
            # speculative step: k drafts get slots and KV, the verifier keeps j
            sid = live[int(rng.integers(len(live)))]
            L0, ok = bm.lens[sid], 0
            try:
                for _ in range(int(rng.integers(1, 5))):
                    append(sid, int(rng.integers(0, 4)))
                    ok += 1
            except BMError:
                pass
            j = int(rng.integers(0, ok + 1))
            rec("truncate", sid, L0 + j)
            bm.truncate(sid, L0 + j)
            del toks[sid][L0 + j:]
        for s in live:
            t = bm.tables[s]
            for p in range(bm.lens[s]):
                assert content.get(t[p // B] * B + p % B) == tuple(toks[s][:p + 1]), (s, p)
        check_invariants(bm)
    return hits


@pytest.mark.parametrize("seed", range(12))
def test_speculative_content_simulation(seed):
    simulate_speculative(1600 + seed)


def test_simulation_reaches_the_cache():
    assert sum(simulate_speculative(1600 + s) for s in range(12)) > 0
