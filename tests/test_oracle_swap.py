"""Pins for swapping in the reference block manager (CPU only).

The pages: a request's KV blocks can be swapped to CPU memory and brought back
("PagedAttention: The vLLM Paper", "The Core Idea", OS-paging analogy table,
"Swapping"; "Implementation Essentials", preemption).  What swapping must
preserve is fixed by that: a sequence that comes back finds exactly its own
tokens.  The pins are a hand-worked example of the FIFO bookkeeping, the
shared-block case, and a content simulation over random scripts in which every
slot of both pools carries a (writer, position) label and every op runs its
copies as a step would."""
import numpy as np
import pytest

from oracle.block_manager import (BlockManager, BMError, EEXIST, EINVAL, ENOBLOCKS, ENOSEQ, OK,
                                  run_ops)
from tests.test_oracle_block_manager import check_invariants
from workloads import random_script


def test_swap_worked_example():
    """Hand-worked: B=2, 4 device blocks, 3 host blocks."""
    bm = BlockManager(4, 2)
    bm.set_host_pool(3)
    bm.add_seq(0, 3)                                # device blocks [0, 1]
    bm.add_seq(1, 2)                                # device block [2]
    assert bm.swap_out(0) == [(0, 0), (1, 1)]       # host blocks 0, 1
    assert list(bm.free) == [3, 0, 1] and list(bm.host_free) == [2]
    assert bm.is_swapped(0) and bm.seq_info(0) == (3, 2)
    for call in (lambda: bm.append_slot(0), lambda: bm.fork(0, 5),
                 lambda: bm.fill_batch([0], 4), lambda: bm.block_table(0)):
        with pytest.raises(BMError) as e:
            call()
        assert e.value.code == EINVAL
    with pytest.raises(BMError) as e:
        bm.swap_in(1)                               # resident, not swapped
    assert e.value.code == EINVAL
    assert bm.swap_out(1) == [(2, 2)]               # the last host block
    with pytest.raises(BMError) as e:
        bm.add_seq(0, 1)                            # the id is still taken
    assert e.value.code == EEXIST
    bm.add_seq(2, 8)                                # takes every device block: [3, 0, 1, 2]
    with pytest.raises(BMError) as e:
        bm.swap_in(0)                               # needs 2 free device blocks
    assert e.value.code == ENOBLOCKS
    assert bm.is_swapped(0) and list(bm.host_free) == []
    bm.free_seq(2)                                  # device free queue [3, 0, 1, 2]
    assert bm.swap_in(1) == [(2, 3)]
    assert bm.swap_in(0) == [(0, 0), (1, 1)]
    assert list(bm.host_free) == [2, 0, 1] and list(bm.free) == [2]
    assert bm.block_table(0) == [0, 1] and bm.block_table(1) == [3]
    assert bm.swap_out(1) == [(3, 2)]
    bm.free_seq(1)                                  # a swapped sequence frees its host blocks
    assert list(bm.host_free) == [0, 1, 2] and list(bm.free) == [2, 3]
    with pytest.raises(BMError) as e:
        bm.swap_out(7)
    assert e.value.code == ENOSEQ


def test_host_pool_is_set_once():
    bm = BlockManager(4, 2)
    with pytest.raises(BMError):
        bm.set_host_pool(0)
    bm.set_host_pool(2)
    with pytest.raises(BMError):
        bm.set_host_pool(2)
    bm.add_seq(0, 4)
    bm.add_seq(1, 1)
    with pytest.raises(BMError) as e:
        bm.swap_out(0)                              # 2 blocks fit the 2 host blocks...
        bm.swap_out(1)                              # ...and then nothing is left
    assert e.value.code == ENOBLOCKS


def test_swap_of_a_shared_block_keeps_the_other_owner():
    """A forked sequence swapped out takes private host copies; the sharer
    keeps the device blocks, and the swapped one returns to private blocks."""
    bm = BlockManager(6, 4)
    bm.set_host_pool(6)
    bm.add_seq(0, 6)                                # [0, 1]
    bm.fork(0, 1)
    assert bm.swap_out(1) == [(0, 0), (1, 1)]
    assert bm.refcount(0) == 1 and bm.refcount(1) == 1 and bm.num_free() == 4
    assert bm.swap_in(1) == [(0, 2), (1, 3)]
    assert bm.block_table(0) == [0, 1] and bm.block_table(1) == [2, 3]
    slot, src, dst = bm.append_slot(1)              # private now: written in place
    assert (src, dst) == (-1, -1) and slot == 3 * 4 + 2


class Contents:
    """What each slot of the device and host pools holds: every written token
    is labelled (sequence that wrote it, position).  Ops run their copies in
    the order a step runs them, so after every op each known sequence must find
    exactly its own tokens through its table, on whichever side it lives."""

    def __init__(self, bm):
        self.bm = bm
        self.dev = [[None] * bm.B for _ in range(bm.N)]
        self.host = [[None] * bm.B for _ in range(bm.NH)]
        self.want = {}                              # seq id -> labels of its tokens

    def apply(self, op, code, result):
        if code != OK:
            return
        B, kind, sid = self.bm.B, op[0], op[1]
        if kind == "add":
            self.want[sid] = [(sid, t) for t in range(op[2])]
            for t, lab in enumerate(self.want[sid]):
                self.dev[self.bm.tables[sid][t // B]][t % B] = lab
        elif kind == "fork":
            self.want[op[2]] = list(self.want[sid])
        elif kind == "append":
            slot, src, dst = result
            if src >= 0:
                self.dev[dst] = list(self.dev[src])
            t = len(self.want[sid])
            self.want[sid].append((sid, t))
            self.dev[slot // B][slot % B] = (sid, t)
        elif kind == "free":
            del self.want[sid]
        elif kind == "swap_out":
            for d, h in result:
                self.host[h] = list(self.dev[d])
        elif kind == "swap_in":
            for h, d in result:
                self.dev[d] = list(self.host[h])

    def check(self):
        B = self.bm.B
        for sid, labels in self.want.items():
            swapped = sid in self.bm.host_tables
            table = self.bm.host_tables[sid] if swapped else self.bm.tables[sid]
            pool = self.host if swapped else self.dev
            assert self.bm.lens[sid] == len(labels)
            for t, lab in enumerate(labels):
                assert pool[table[t // B]][t % B] == lab, (sid, t, swapped)


def check_host_invariants(bm):
    used = [h for t in bm.host_tables.values() for h in t]
    free = list(bm.host_free)
    assert len(used) == len(set(used)) and len(free) == len(set(free))
    assert sorted(used + free) == list(range(bm.NH))
    for sid, t in bm.host_tables.items():
        assert len(t) == -(-bm.lens[sid] // bm.B)
        assert sid not in bm.tables


def _state(bm):
    return (bm.snapshot(), list(bm.host_free), {k: list(v) for k, v in bm.tables.items()},
            {k: list(v) for k, v in bm.host_tables.items()}, dict(bm.lens))


def _run_swap_script(seed):
    rng = np.random.default_rng(7000 + seed)
    N, B = int(rng.integers(4, 40)), int(rng.choice([1, 2, 4, 16]))
    NH = int(rng.integers(1, 40))
    bm = BlockManager(N, B, rng.permutation(N))
    bm.set_host_pool(NH)
    mem = Contents(bm)
    swaps = 0
    for op in random_script(rng, 400, max_seqs=6, max_add=5 * B, swap=True):
        before = _state(bm)
        resident, swapped = op[1] in bm.tables, op[1] in bm.host_tables
        nfree, nhost = bm.num_free(), bm.num_free_host()
        codes, res = run_ops(bm, [op])
        if codes[0] != OK:      # every failing call leaves the state unchanged
            assert _state(bm) == before
        if op[0] == "swap_out" and resident:
            # all or nothing: succeeds iff the host has a block per table entry
            assert (codes[0] == OK) == (nhost >= len(before[2][op[1]]))
        if op[0] == "swap_in" and swapped:
            assert (codes[0] == OK) == (nfree >= len(before[3][op[1]]))
        if op[0] in ("swap_out", "swap_in"):
            if not (resident or swapped):
                assert codes[0] == ENOSEQ
            swaps += codes[0] == OK
        mem.apply(op, codes[0], res[0] if res else None)
        mem.check()
        check_invariants(bm)
        check_host_invariants(bm)
    for sid in list(bm.tables) + list(bm.host_tables):
        bm.free_seq(sid)
    assert bm.num_free() == N and bm.num_free_host() == NH
    return swaps


@pytest.mark.parametrize("seed", range(40))
def test_swap_random_scripts_keep_every_sequence_content(seed):
    _run_swap_script(seed)


def test_swap_random_scripts_do_swap():
    assert sum(_run_swap_script(seed) > 0 for seed in range(40)) >= 30
