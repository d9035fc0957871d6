"""Pins for the reference block manager (CPU only).

Worked facts from the pages, the block-pool figure, and the OS-paging
invariants, checked after every op of many seeded random scripts."""
import json
import os

import numpy as np
import pytest

from oracle.block_manager import (BlockManager, BMError, EEXIST, ENOBLOCKS, ENOSEQ, OK,
                                  run_ops)
from workloads import random_script

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_example_70_tokens():
    g = _golden("worked_example_70_tokens.json")
    B = g["block_size"]
    bm = BlockManager(16, B)
    bm.add_seq(0, g["tokens"])
    L, nb = bm.seq_info(0)
    assert nb == g["blocks"]
    assert L - (nb - 1) * B == g["used_slots_in_last_block"]
    assert sum(1 for j in range(nb) if (j + 1) * B <= L) == g["full_blocks"]
    # the same state reached one token at a time
    bm.add_seq(1, 0)
    for _ in range(g["tokens"]):
        bm.append_slot(1)
    assert bm.seq_info(1) == (g["tokens"], g["blocks"])
    # waste bound: never more than B-1 empty slots, for any length
    for n in range(0, 300):
        nb = -(-n // B)
        assert nb * B - n <= g["max_wasted_slots_per_request"]


def test_block_pool_figure():
    g = _golden("block_pool_figure.json")
    B = g["block_size"]
    bm = BlockManager(g["num_blocks"], B)
    ids = {"A": 0, "B": 1, "C": 2, "D": 3}

    def take_one(name):
        sid = ids[name]
        if sid not in bm.tables:
            bm.add_seq(sid, B)          # first block, full
        else:
            for _ in range(B):          # the first of B appends opens a new block
                bm.append_slot(sid)

    for name in "ABACBCAB":
        take_one(name)
    bm.free_seq(ids["C"])
    assert bm.block_table(ids["A"]) == g["tables"]["A"]
    assert bm.block_table(ids["B"]) == g["tables"]["B"]
    assert sorted(bm.free) == g["empty_blocks"]
    # returned blocks are reusable by any request
    bm.add_seq(ids["D"], 2 * B)
    assert bm.block_table(ids["D"]) == g["empty_blocks"]
    assert bm.num_free() == 0


def check_invariants(bm: BlockManager):
    N, B = bm.N, bm.B
    counts = [0] * N
    for sid, t in bm.tables.items():
        L = bm.lens[sid]
        assert len(t) == -(-L // B)                         # I3: ceil(len/B) blocks
        assert len(t) * B - L <= B - 1                      # I3: only the last is partial
        for b in t:
            counts[b] += 1
    assert counts == bm.ref                                 # I1
    free = list(bm.free)
    assert len(free) == len(set(free))                      # I2: no duplicates
    assert set(free) == {b for b in range(N) if bm.ref[b] == 0}   # I2


@pytest.mark.parametrize("seed", range(40))
def test_invariants_random_scripts(seed):
    rng = np.random.default_rng(1000 + seed)
    N, B = int(rng.integers(4, 40)), int(rng.choice([1, 2, 4, 16]))
    bm = BlockManager(N, B, rng.permutation(N))
    for op in random_script(rng, 300, max_seqs=6, max_add=5 * B):
        before = (bm.snapshot(), {k: list(v) for k, v in bm.tables.items()}, dict(bm.lens))
        kind = op[0]
        nfree = bm.num_free()
        codes, appends = run_ops(bm, [op])
        if codes[0] != OK:      # every failing call leaves the state unchanged
            assert (bm.snapshot(), bm.tables, bm.lens) == before
        if kind == "add" and op[1] not in before[1]:
            # I4: admission succeeds iff enough blocks are free
            assert (codes[0] == OK) == (nfree >= -(-op[2] // B))
        if kind == "append" and codes[0] == OK:
            slot, src, dst = appends[0]
            t = bm.tables[op[1]]
            L = bm.lens[op[1]]
            assert slot == t[(L - 1) // B] * B + (L - 1) % B
            assert bm.ref[t[(L - 1) // B]] == 1                 # I5: the written block is private
            if src >= 0:
                assert dst == t[-1] and src not in t
        check_invariants(bm)
    # I6: finishing every sequence returns the whole pool
    for sid in list(bm.tables):
        bm.free_seq(sid)
    assert bm.num_free() == N and all(r == 0 for r in bm.ref)


def test_copy_on_write_fork():
    B = 16
    bm = BlockManager(32, B)
    bm.add_seq(0, 20)                       # blocks [0, 1], last holds 4 tokens
    for c in (1, 2, 3):
        bm.fork(0, c)
    assert bm.refcount(0) == 4 and bm.refcount(1) == 4
    pairs = []
    for sid in (0, 1, 2, 3):
        slot, src, dst = bm.append_slot(sid)
        pairs.append((src, dst))
        assert slot == bm.block_table(sid)[1] * B + 4
    # the first three writers copy the shared partial block; the last writes in place
    assert [p[0] for p in pairs] == [1, 1, 1, -1]
    assert [p[1] for p in pairs[:3]] == [2, 3, 4]
    assert bm.block_table(3) == [0, 1] and bm.refcount(1) == 1
    assert bm.refcount(0) == 4              # the full shared block is untouched


def test_full_shared_block_is_not_copied():
    B = 16
    bm = BlockManager(8, B)
    bm.add_seq(0, 32)
    bm.fork(0, 1)
    slot, src, dst = bm.append_slot(1)
    assert (src, dst) == (-1, -1)
    assert bm.block_table(1) == [0, 1, 2] and slot == 2 * B
    assert bm.refcount(1) == 2


def test_error_paths_leave_state_unchanged():
    bm = BlockManager(4, 16)
    bm.add_seq(0, 40)                      # 3 blocks
    snap = bm.snapshot()
    with pytest.raises(BMError) as e:
        bm.add_seq(1, 40)
    assert e.value.code == ENOBLOCKS and bm.snapshot() == snap
    with pytest.raises(BMError) as e:
        bm.add_seq(0, 1)
    assert e.value.code == EEXIST
    with pytest.raises(BMError) as e:
        bm.append_slot(7)
    assert e.value.code == ENOSEQ
    with pytest.raises(BMError) as e:
        bm.fork(0, 0)
    assert e.value.code == EEXIST
    bm.fork(0, 1)
    # CoW needs a free block: one left, so the first copy succeeds, the second fails
    bm.fork(0, 2)
    bm.append_slot(0)
    snap = (bm.snapshot(), {k: list(v) for k, v in bm.tables.items()})
    with pytest.raises(BMError) as e:
        bm.append_slot(1)
    assert e.value.code == ENOBLOCKS
    assert (bm.snapshot(), bm.tables) == snap
    bm.free_seq(2)
    with pytest.raises(BMError) as e:
        bm.free_seq(2)                     # double free
    assert e.value.code == ENOSEQ


def test_count_shared_follows_fork_and_cow():
    """Forked samples reference the parent's blocks ("Pages, from operating
    systems": sequences that share a prefix map to the same physical blocks) and
    a shared block stops being shared once each writer has its own copy."""
    from oracle.block_manager import count_shared
    bm = BlockManager(16, 16)
    bm.add_seq(0, 50)                  # 3 full blocks + 1 holding 2 tokens
    for child in (1, 2, 3):
        bm.fork(0, child)
    assert count_shared(bm, [0, 1, 2, 3]) == 4 * 4
    for sid in (0, 1, 2, 3):           # 0, 1, 2 copy the partial block; 3 writes in place
        bm.append_slot(sid)
    assert count_shared(bm, [0, 1, 2, 3]) == 4 * 3
    for sid in (1, 2, 3):
        bm.free_seq(sid)
    assert count_shared(bm, [0]) == 0

