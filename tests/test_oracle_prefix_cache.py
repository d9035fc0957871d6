"""Pins for prefix caching in the reference block manager (CPU only).

The pages: the KV of a shared prompt prefix is cached and reused across
requests, so on a hit that part of the prefill is free ("PagedAttention: The
vLLM Paper", "Impact and Follow-Ups"; "Implementation Essentials", prefix
sharing).  What must hold: a reused block holds exactly the KV the new request
would have written.  Pinned by a hand-worked example and by a content
simulation over random scripts in which every slot is labelled with the whole
token prefix up to it (the KV of a token depends on every token before it), so
a block reused for a different prefix shows up at once."""
import numpy as np
import pytest

from oracle.block_manager import BlockManager, BMError, EEXIST, EINVAL, ENOBLOCKS
from tests.test_oracle_block_manager import check_invariants


def admit(bm, sid, tokens, n):
    """Admission as a caller does it: reuse cached blocks, then register the
    full blocks it is about to write."""
    cached = bm.add_seq_prefix(sid, tokens, n)
    bm.register_prefix(sid, tokens, n)
    return cached


def test_prefix_cache_worked_example():
    """B=4, 8 blocks, FIFO free queue 0..7."""
    bm = BlockManager(8, 4)
    a = list(range(1, 11))                               # 10 tokens: blocks [0, 1, 2]
    assert admit(bm, 0, a, 10) == 0              # nothing cached yet
    assert bm.tables[0] == [0, 1, 2] and bm.cached_blocks() == 2
    b = list(range(1, 9)) + [99, 98, 97]                 # same first 8 tokens
    assert admit(bm, 1, b, 11) == 8              # blocks 0 and 1 reused
    assert bm.tables[1] == [0, 1, 3] and bm.refcount(0) == 2 and bm.refcount(1) == 2
    c = [1, 2, 3, 4, 50, 51]                             # first block only
    assert admit(bm, 2, c, 6) == 4
    assert bm.tables[2] == [0, 4] and bm.refcount(0) == 3
    # a different first block shares nothing, even with equal later tokens
    d = [7, 2, 3, 4] + list(range(5, 9))
    assert admit(bm, 3, d, 8) == 0 and bm.tables[3] == [5, 6]
    # free everything, each table walked from block 0: the cached blocks stay
    # cached in the free queue
    for sid in (0, 1, 2, 3):
        bm.free_seq(sid)
    assert list(bm.free) == [7, 2, 1, 3, 0, 4, 5, 6] and bm.cached_blocks() == 4
    # a whole cached prompt still leaves its last block to compute: of a's first
    # 8 tokens only block 0 is reused, and it comes back out of the free queue
    assert admit(bm, 4, a[:8], 8) == 4
    assert bm.tables[4] == [0, 7] and list(bm.free) == [2, 1, 3, 4, 5, 6]
    # taking blocks from the queue front evicts what they cached: block 1 (a's
    # 8-token prefix)
    bm.add_seq(5, 8)
    assert bm.tables[5] == [2, 1] and bm.cached_blocks() == 3
    # a hits block 0 (in use by sequence 4), misses its evicted second block,
    # and registers the fresh block 3 for that prefix
    assert admit(bm, 6, a, 10) == 4
    assert bm.tables[6] == [0, 3, 4] and bm.refcount(0) == 2 and bm.cached_blocks() == 4
    # d hits block 5 from the free queue; its fresh second block is block 6,
    # whose own cached entry (d's 8-token prefix) is evicted and registered again
    assert admit(bm, 7, d, 8) == 4
    assert bm.tables[7] == [5, 6] and list(bm.free) == [] and bm.cached_blocks() == 4


def test_prefix_cache_is_all_or_nothing():
    bm = BlockManager(3, 4)
    admit(bm, 0, list(range(8)), 8)              # blocks [0, 1], both cached
    bm.free_seq(0)                                       # free queue [2, 0, 1]
    before = (bm.snapshot(), dict(bm.cache), dict(bm.cached_key))
    # 4 cached tokens hit block 0 (taken out of the queue); 3 more blocks needed
    with pytest.raises(BMError) as e:
        bm.add_seq_prefix(1, list(range(8)) + [9] * 8, 16)
    assert e.value.code == ENOBLOCKS
    assert (bm.snapshot(), dict(bm.cache), dict(bm.cached_key)) == before
    with pytest.raises(BMError) as e:
        bm.add_seq_prefix(1, list(range(8)), 5)          # fewer tokens than known ids
    assert e.value.code == EINVAL
    bm.add_seq(2, 1)
    with pytest.raises(BMError) as e:
        bm.add_seq_prefix(2, [0], 1)
    assert e.value.code == EEXIST


def check_cache_invariants(bm):
    assert len(bm.cache) == len(bm.cached_key)
    for key, b in bm.cache.items():
        assert bm.cached_key[b] == key
        assert len(key) % bm.B == 0 and key


class Labels:
    """Every slot holds the label of the whole token prefix up to it; the
    sequences' token ids are known (prompts) or made unique (generated)."""

    def __init__(self, bm):
        self.bm = bm
        self.pool = [[None] * bm.B for _ in range(bm.N)]
        self.toks = {}

    def admit(self, sid, tokens, n, cached):
        t = list(tokens) + [("gen", sid, i) for i in range(len(tokens), n)]
        self.toks[sid] = t
        tab = self.bm.tables[sid]
        for i in range(cached, n):                       # the caller writes the rest
            self.pool[tab[i // self.bm.B]][i % self.bm.B] = tuple(t[:i + 1])

    def append(self, sid, slot, src, dst):
        if src >= 0:
            self.pool[dst] = list(self.pool[src])
        t = self.toks[sid]
        t.append(("gen", sid, len(t)))
        self.pool[slot // self.bm.B][slot % self.bm.B] = tuple(t)

    def check(self):
        B = self.bm.B
        for sid, t in self.toks.items():
            tab = self.bm.tables[sid]
            for i in range(len(t)):
                assert self.pool[tab[i // B]][i % B] == tuple(t[:i + 1]), (sid, i)


def run_prefix_script(seed, bm_cls=BlockManager):
    rng = np.random.default_rng(5100 + seed)
    B = int(rng.choice([1, 2, 4, 16]))
    N = int(rng.integers(6, 60))
    bm = bm_cls(N, B, rng.permutation(N))
    lab = Labels(bm)
    prompts = [list(rng.integers(0, 3, size=int(rng.integers(1, 6 * B)))) for _ in range(4)]
    hits = 0
    for _ in range(300):
        sid = int(rng.integers(0, 6))
        r = rng.random()
        if r < 0.35:
            base = prompts[int(rng.integers(0, len(prompts)))]
            cut = int(rng.integers(0, len(base) + 1))
            tokens = base[:cut] + list(rng.integers(0, 3, size=int(rng.integers(0, 2 * B))))
            n = len(tokens) + int(rng.integers(0, B + 1))
            before = (bm.snapshot(), dict(bm.cache))
            nfree = bm.num_free()
            try:
                cached = bm.add_seq_prefix(sid, tokens, n)
            except BMError as e:
                assert (bm.snapshot(), dict(bm.cache)) == before
                if e.code == ENOBLOCKS:
                    assert nfree < -(-n // B)            # could not have fit without hits
                continue
            assert cached % B == 0 and cached <= max(n - 1, 0)
            hits += cached > 0
            lab.admit(sid, tokens, n, cached)
            bm.register_prefix(sid, tokens, n)
        elif r < 0.85:
            if sid in bm.tables:
                try:
                    slot, src, dst = bm.append_slot(sid)
                except BMError:
                    continue
                lab.append(sid, slot, src, dst)
        elif r < 0.92 and sid in bm.tables:
            child = int(rng.integers(0, 6))
            if child not in bm.tables:
                bm.fork(sid, child)
                lab.toks[child] = list(lab.toks[sid])
        elif sid in bm.tables:
            bm.free_seq(sid)
            del lab.toks[sid]
        lab.check()
        check_invariants(bm)
        check_cache_invariants(bm)
    return hits


@pytest.mark.parametrize("seed", range(30))
def test_prefix_cache_keeps_every_sequence_content(seed):
    run_prefix_script(seed)


def test_random_scripts_do_hit():
    assert sum(run_prefix_script(s) > 0 for s in range(30)) >= 20


def test_registration_and_withdrawal():
    """Admission alone registers nothing; registration covers full blocks up to
    the given token; withdrawal drops the sequence's own entries past a token
    and keeps reused ones."""
    bm = BlockManager(10, 4)
    t = list(range(12))
    assert bm.add_seq_prefix(0, t, 12) == 0 and bm.cached_blocks() == 0
    bm.register_prefix(0, t, 6)                          # only block 0 is full by token 6
    assert bm.cached_blocks() == 1
    bm.register_prefix(0, t, 12)
    assert bm.cached_blocks() == 3
    assert bm.add_seq_prefix(1, t[:8] + [40], 9) == 8     # reuses blocks 0, 1
    bm.unregister_prefix(1, 8)                           # its own third block was never cached
    assert bm.cached_blocks() == 3
    bm.unregister_prefix(0, 5)                           # blocks 1, 2 of sequence 0: 1 is shared
    assert bm.cached_blocks() == 2 and bm.tables[0][2] not in bm.cached_key
    with pytest.raises(BMError):
        bm.register_prefix(0, t, 13)
