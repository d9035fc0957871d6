"""Pins for the reference's slot rule and valid-slot mask (CPU only).

The pages place a sequence's token t in logical block t // B of its block
table, at offset t % B inside that block ("PagedAttention and Continuous
Batching", "Pages, from operating systems"; "PagedAttention: The vLLM Paper",
"The Core Idea", block-pool figure).  `oracle.block_manager.slots` computes the
slots of a token range from the table, and `oracle.attention.valid_slot_mask`
marks which pool slots hold a token.  Both are pinned here against facts that
do not go through them:

  * the history of writes: every token's slot is the one `append_slot` returned
    when the token was written, moved to the destination block whenever a
    copy-on-write copied its block (the copy keeps offsets), inherited by a
    fork and dropped by a truncation;
  * the block-pool figure: request A's 48 tokens sit in blocks 0, 2 and 6 and
    B's in 1, 4 and 7, blocks 3 and 5 hold nothing;
  * counting: over private tables the mask marks exactly sum(L) slots.
"""
import json
import os

import numpy as np
import pytest

from oracle.attention import valid_slot_mask
from oracle.block_manager import BlockManager, BMError, slots

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _figure():
    with open(os.path.join(GOLDEN, "block_pool_figure.json")) as f:
        return json.load(f)


def _figure_state(g):
    """The figure's final state, reached as the block-manager pins reach it: A, B,
    A, C, B, C, A, B each take one block from an ascending free queue, then C
    finishes."""
    B = g["block_size"]
    bm = BlockManager(g["num_blocks"], B)
    ids = {"A": 0, "B": 1, "C": 2}
    for name in "ABACBCAB":
        sid = ids[name]
        if sid not in bm.tables:
            bm.add_seq(sid, 0)
        for _ in range(B):
            bm.append_slot(sid)
    bm.free_seq(ids["C"])
    return bm, ids


def test_slots_on_block_pool_figure():
    g = _figure()
    B = g["block_size"]
    bm, ids = _figure_state(g)
    for name in ("A", "B"):
        want = [b * B + o for b in g["tables"][name] for o in range(B)]
        assert slots(bm, ids[name], 0, 3 * B) == want
        # any sub-range is the matching slice
        assert slots(bm, ids[name], B - 1, B + 2) == want[B - 1:2 * B + 1]
        assert slots(bm, ids[name], 3 * B, 0) == []
    # five more tokens of A open a fourth block: the first empty one the free
    # queue hands out, filled from offset 0
    empty = g["empty_blocks"]
    written = [bm.append_slot(ids["A"])[0] for _ in range(5)]
    assert slots(bm, ids["A"], 3 * B, 5) == written
    assert {s // B for s in written} <= set(empty)
    assert [s % B for s in written] == list(range(5))
    with pytest.raises(BMError):
        slots(bm, ids["A"], 3 * B, 6)          # past the sequence's length


def test_valid_slot_mask_on_block_pool_figure():
    g = _figure()
    B, N = g["block_size"], g["num_blocks"]
    bm, ids = _figure_state(g)
    tables, lens = bm.fill_batch([ids["A"], ids["B"]], 4)
    mask = valid_slot_mask(tables, lens, N, B)
    for b in range(N):
        assert mask[b].all() == (b not in g["empty_blocks"])
        assert mask[b].any() == (b not in g["empty_blocks"])
    # a partial last block: exactly its first five slots hold tokens
    for _ in range(5):
        bm.append_slot(ids["A"])
    tables, lens = bm.fill_batch([ids["A"], ids["B"]], 4)
    mask = valid_slot_mask(tables, lens, N, B)
    opened = bm.block_table(ids["A"])[3]
    assert mask[opened].tolist() == [True] * 5 + [False] * (B - 5)
    assert int(mask.sum()) == sum(lens)


@pytest.mark.parametrize("seed", range(12))
def test_valid_slot_mask_counts_private_tokens(seed):
    """With no shared blocks, every token has its own slot: the mask marks exactly
    sum(L) slots, and a block's marked slots are a prefix of it."""
    rng = np.random.default_rng(500 + seed)
    B = int(rng.choice([1, 2, 4, 16, 32]))
    lens = [int(x) for x in rng.integers(0, 5 * B, size=int(rng.integers(1, 7)))]
    N = sum(-(-L // B) for L in lens) + int(rng.integers(0, 4))
    bm = BlockManager(max(N, 1), B, rng.permutation(max(N, 1)))
    for s, L in enumerate(lens):
        bm.add_seq(s, L)
    maxb = max(1, max(-(-L // B) for L in lens))
    tables, clens = bm.fill_batch(range(len(lens)), maxb)
    mask = valid_slot_mask(tables, clens, max(N, 1), B)
    assert int(mask.sum()) == sum(lens)
    for row in mask:
        n = int(row.sum())
        assert row[:n].all() and not row[n:].any()


def _apply_cow(hist, B, src, dst):
    """A copy-on-write copy moves this writer's tokens of block src to dst at the
    same offsets."""
    return [dst * B + s % B if s // B == src else s for s in hist]


@pytest.mark.parametrize("seed", range(30))
def test_slots_equal_append_history(seed):
    """Random token-by-token scripts with forks, frees and truncations: slots()
    of every live sequence equals the slots its tokens were written to."""
    rng = np.random.default_rng(900 + seed)
    B = int(rng.choice([1, 2, 4, 16]))
    N = int(rng.integers(6, 48))
    bm = BlockManager(N, B, rng.permutation(N))
    hist = {}
    next_id = 0
    for _ in range(250):
        live = sorted(hist)
        r = rng.random()
        try:
            if r < 0.12 or not live:
                bm.add_seq(next_id, 0)
                hist[next_id] = []
                next_id += 1
            elif r < 0.70:
                s = live[int(rng.integers(len(live)))]
                for _ in range(int(rng.integers(1, 2 * B + 2))):
                    slot, src, dst = bm.append_slot(s)
                    if src >= 0:
                        hist[s] = _apply_cow(hist[s], B, src, dst)
                    hist[s].append(slot)
            elif r < 0.82:
                s = live[int(rng.integers(len(live)))]
                bm.fork(s, next_id)
                hist[next_id] = list(hist[s])
                next_id += 1
            elif r < 0.92:
                s = live[int(rng.integers(len(live)))]
                n = int(rng.integers(0, len(hist[s]) + 1))
                bm.truncate(s, n)
                hist[s] = hist[s][:n]
            else:
                s = live[int(rng.integers(len(live)))]
                bm.free_seq(s)
                del hist[s]
        except BMError:
            pass                      # a failed call changes nothing (pinned elsewhere)
        for s, h in hist.items():
            assert bm.seq_info(s)[0] == len(h)
            assert slots(bm, s, 0, len(h)) == h
            if h:
                a = int(rng.integers(len(h)))
                c = int(rng.integers(len(h) - a + 1))
                assert slots(bm, s, a, c) == h[a:a + c]
