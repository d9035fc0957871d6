"""Reference host block manager.

From the pages:
  * the KV cache is split into fixed-size blocks (16 tokens by default) and each
    request's logical blocks map to physical ones through a block table; blocks
    are allocated as tokens are generated ("PagedAttention and Continuous
    Batching", "The solution", "Pages, from operating systems");
  * worked example: 70 tokens at 16 tokens per block hold 5 blocks, the last
    with 6 of 16 slots used; at most 15 slots are wasted per request (same
    section);
  * the pool is allocated once; blocks are claimed on demand, returned when
    done and reusable by any request ("PagedAttention: The vLLM Paper", "The
    Core Idea", block-pool figure; "Implementation Essentials");
  * refcounts let sequences share blocks; a shared block is copied only when one
    sharer is about to write it (copy-on-write, as in an OS fork) ("Pages, from
    operating systems"; "The Core Idea", OS-paging analogy table);
  * only the last block of a sequence may be partially filled, and uniform
    blocks leave no external fragmentation ("The Core Idea", three wins).

Readings where the pages are silent:
  * free blocks form a FIFO queue; its initial order is given by the caller
    (ascending by default) and freed blocks are appended in release order,
    walking the freed sequence's table from logical block 0 upward;
  * append_slot on a sequence whose length is a multiple of B allocates a new
    private block (a full shared block is never written, so it is not copied);
    otherwise, if its last block is shared (refcount > 1), a new block is
    allocated, the pair (src, dst) is emitted for the device copy, src loses one
    reference and dst replaces it in the table; a last block with refcount 1 is
    written in place;
  * add_seq(n) is all-or-nothing: it fails with no change when fewer than
    ceil(n/B) blocks are free; every failing call leaves the state unchanged.

Swapping ("The Core Idea", OS-paging analogy table, "Swapping": KV blocks go
to CPU memory; "Implementation Essentials": preemption swaps a request's
blocks to the CPU).  Readings where the pages are silent:
  * a host pool of blocks with the device pool's geometry, set once; its free
    blocks form a FIFO queue, initially ascending;
  * swap_out(s) moves a resident sequence to the host: walking its table from
    logical block 0 it takes one host block per table entry (pairs (device
    block, host block) for the copy), then releases its device blocks as
    free_seq does.  A block the sequence shares keeps its other references on
    the device; the host copy is private to the swapped sequence;
  * swap_in(s) brings it back: one new device block per host block, in table
    order (pairs (host block, device block)), then the host blocks return to
    the host free queue in table order;
  * both are all-or-nothing (too few free blocks on the destination side:
    ENOBLOCKS, no change); a swapped sequence cannot be appended to, forked or
    batched (EINVAL) but can be freed, and keeps its length.

Speculative drafts ("Impact and Follow-Ups": multi-token queries over paged
KV also serve speculative decoding): draft tokens take slots through
append_slot like any token, and truncate(s, n) gives back those a verification
rejects.  Readings where the pages are silent: the blocks past ceil(n/B) are
released in logical order as free_seq releases them; the kept last block, when
it becomes partial and is not shared, loses its prefix-cache entry (its slots
past n will be rewritten); truncating to a length the sequence already has
changes nothing.

Prefix caching ("Impact and Follow-Ups": the KV of a shared prompt prefix is
cached and reused across requests, so a hit makes that part of the prefill
free; "Implementation Essentials": prefix sharing through block refcounts).
Readings where the pages are silent:
  * a full block's content is identified by the token ids of the whole prefix
    up to its end (exact: no hash collisions can merge different prefixes);
  * add_seq_prefix(s, tokens, n) admits a sequence of n tokens whose first
    len(tokens) ids are known: walking its full blocks from logical block 0 it
    reuses the cached block of each prefix while one exists (refcount + 1; a
    cached block with refcount 0 is taken back out of the free queue), at most
    (n - 1) // B blocks, so at least one token is always left to compute; the
    rest are fresh blocks as in add_seq.  Returns the number of cached tokens;
  * register_prefix(s, tokens, upto) registers each full block of the
    sequence that the known ids cover and that ends at or before token `upto`,
    unless another block already holds that prefix: the caller calls it once
    that KV is written or about to be written before anything reads it (a
    prefill chunk); unregister_prefix(s, start) withdraws the sequence's own
    entries for blocks that end after token `start` (KV that will not be
    written after all);
  * a block stays cached while it is in use and after it is freed, until it is
    taken from the free queue for other content (the queue order then makes
    the least recently freed cached block the first to go);
  * all-or-nothing: ENOBLOCKS when the free queue, after the hits are taken out
    of it, holds fewer blocks than the rest needs.
"""
from __future__ import annotations

from collections import deque

OK, EINVAL, ENOBLOCKS, ENOSEQ, EEXIST = 0, -1, -2, -3, -4


class BMError(Exception):
    def __init__(self, code: int, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, init_free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise BMError(EINVAL, "num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if init_free_order is None else [int(b) for b in init_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise BMError(EINVAL, "initial free order must be a permutation of the pool")
        self.N = num_blocks
        self.B = block_size
        self.ref = [0] * num_blocks
        self.free = deque(order)
        self.tables = {}   # seq id -> list of physical block ids
        self.lens = {}     # seq id -> tokens held
        self.cache = {}              # prefix token ids (tuple) -> block holding them
        self.cached_key = {}         # block -> its prefix key, while cached
        self.NH = 0                  # host pool blocks
        self.host_free = deque()
        self.host_tables = {}        # swapped seq id -> list of host block ids

    # -- queries -------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, block: int) -> int:
        if not 0 <= block < self.N:
            raise BMError(EINVAL, "block out of range")
        return self.ref[block]

    def seq_info(self, sid: int):
        if not self._known(sid):
            raise BMError(ENOSEQ)
        t = self.tables[sid] if sid in self.tables else self.host_tables[sid]
        return self.lens[sid], len(t)

    def block_table(self, sid: int):
        self._resident(sid)
        return list(self.tables[sid])

    def _resident(self, sid: int) -> None:
        if sid in self.host_tables:
            raise BMError(EINVAL, "sequence is swapped out")
        if sid not in self.tables:
            raise BMError(ENOSEQ)

    def _known(self, sid: int) -> bool:
        return sid in self.tables or sid in self.host_tables

    def is_swapped(self, sid: int) -> bool:
        if not self._known(sid):
            raise BMError(ENOSEQ)
        return sid in self.host_tables

    def num_free_host(self) -> int:
        return len(self.host_free)

    def snapshot(self):
        return list(self.ref), list(self.free)

    # -- updates -------------------------------------------------------------
    def _take(self) -> int:
        b = self.free.popleft()
        self.ref[b] = 1
        key = self.cached_key.pop(b, None)      # reused for other content
        if key is not None:
            del self.cache[key]
        return b

    def add_seq_prefix(self, sid: int, tokens, num_tokens: int) -> int:
        """Admit a sequence whose first len(tokens) token ids are known,
        reusing cached full blocks of its prefix.  Returns the number of tokens
        whose KV is already cached (a multiple of B)."""
        tokens = [int(t) for t in tokens]
        if num_tokens < len(tokens) or num_tokens < 0:
            raise BMError(EINVAL, "num_tokens below the known ids")
        if self._known(sid):
            raise BMError(EEXIST)
        B = self.B
        full = len(tokens) // B                 # full blocks the ids cover
        hits = []
        for j in range(min(full, max(num_tokens - 1, 0) // B)):
            b = self.cache.get(tuple(tokens[:(j + 1) * B]))
            if b is None:
                break
            hits.append(b)
        need = -(-num_tokens // B) - len(hits)
        from_free = sum(1 for b in hits if self.ref[b] == 0)
        if need > len(self.free) - from_free:
            raise BMError(ENOBLOCKS)
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        table = hits + [self._take() for _ in range(need)]
        self.tables[sid] = table
        self.lens[sid] = num_tokens
        return len(hits) * B

    def register_prefix(self, sid: int, tokens, upto: int) -> None:
        self._resident(sid)
        tokens = [int(t) for t in tokens]
        if upto < 0 or upto > self.lens[sid] or len(tokens) > self.lens[sid]:
            raise BMError(EINVAL, "tokens past the sequence's length")
        table, B = self.tables[sid], self.B
        for j in range(min(upto, len(tokens)) // B):
            key = tuple(tokens[:(j + 1) * B])
            if key not in self.cache and table[j] not in self.cached_key:
                self.cache[key] = table[j]
                self.cached_key[table[j]] = key

    def unregister_prefix(self, sid: int, start: int) -> None:
        self._resident(sid)
        if start < 0:
            raise BMError(EINVAL, "negative token index")
        table = self.tables[sid]
        for j in range(start // self.B, len(table)):
            key = self.cached_key.get(table[j])
            if key is not None and self.ref[table[j]] == 1:
                del self.cache[key]
                del self.cached_key[table[j]]

    def cached_blocks(self) -> int:
        return len(self.cache)

    def add_seq(self, sid: int, num_tokens: int) -> None:
        if num_tokens < 0:
            raise BMError(EINVAL, "negative length")
        if self._known(sid):
            raise BMError(EEXIST)
        need = -(-num_tokens // self.B)
        if need > len(self.free):
            raise BMError(ENOBLOCKS)
        self.tables[sid] = [self._take() for _ in range(need)]
        self.lens[sid] = num_tokens

    def append_slot(self, sid: int):
        """Reserve the slot for the sequence's next token.  Returns
        (slot, cow_src, cow_dst); cow_src = cow_dst = -1 when no copy is due."""
        self._resident(sid)
        table, L, B = self.tables[sid], self.lens[sid], self.B
        src = dst = -1
        if L % B == 0:
            if not self.free:
                raise BMError(ENOBLOCKS)
            table.append(self._take())
        else:
            last = table[-1]
            if self.ref[last] > 1:
                if not self.free:
                    raise BMError(ENOBLOCKS)
                dst = self._take()
                self.ref[last] -= 1
                src = last
                table[-1] = dst
        slot = table[L // B] * B + L % B
        self.lens[sid] = L + 1
        return slot, src, dst

    def fork(self, parent: int, child: int) -> None:
        self._resident(parent)
        if self._known(child):
            raise BMError(EEXIST)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, sid: int) -> None:
        if sid in self.host_tables:
            self.host_free.extend(self.host_tables.pop(sid))
            del self.lens[sid]
            return
        if sid not in self.tables:
            raise BMError(ENOSEQ)
        self._release(self.tables.pop(sid))
        del self.lens[sid]

    def truncate(self, sid: int, new_len: int) -> None:
        """Give back the tokens of a resident sequence past new_len (rejected
        speculative draft tokens).  Blocks past ceil(new_len / B) are released
        as free_seq releases them, in logical order; if the kept last block
        becomes partial, later appends will overwrite it in place, so a prefix
        cache entry it holds is withdrawn when no other sequence shares it."""
        self._resident(sid)
        L = self.lens[sid]
        if new_len < 0 or new_len > L:
            raise BMError(EINVAL, "new length outside [0, length]")
        table, B = self.tables[sid], self.B
        keep = -(-new_len // B)
        if new_len % B and self.ref[table[keep - 1]] == 1:
            key = self.cached_key.pop(table[keep - 1], None)
            if key is not None:
                del self.cache[key]
        self._release(table[keep:])
        del table[keep:]
        self.lens[sid] = new_len

    def _release(self, table) -> None:
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- swapping ------------------------------------------------------------
    def set_host_pool(self, num_host_blocks: int) -> None:
        if num_host_blocks <= 0 or self.NH:
            raise BMError(EINVAL, "host pool is set once, with a positive size")
        self.NH = num_host_blocks
        self.host_free = deque(range(num_host_blocks))

    def swap_out(self, sid: int):
        """Move a resident sequence to host blocks; returns the (device block,
        host block) copies, in table order, to run before any write to the
        released device blocks."""
        self._resident(sid)
        table = self.tables[sid]
        if len(table) > len(self.host_free):
            raise BMError(ENOBLOCKS)
        host = [self.host_free.popleft() for _ in table]
        self._release(table)
        del self.tables[sid]
        self.host_tables[sid] = host
        return list(zip(table, host))

    def swap_in(self, sid: int):
        """Bring a swapped sequence back into new device blocks; returns the
        (host block, device block) copies, in table order."""
        if sid not in self.host_tables:
            raise BMError(EINVAL if sid in self.tables else ENOSEQ)
        host = self.host_tables[sid]
        if len(host) > len(self.free):
            raise BMError(ENOBLOCKS)
        table = [self._take() for _ in host]
        self.host_free.extend(host)
        del self.host_tables[sid]
        self.tables[sid] = table
        return list(zip(host, table))

    def fill_batch(self, sids, max_blocks: int):
        """Block tables [n, max_blocks] (padded with -1) and context lengths."""
        tables, lens = [], []
        for sid in sids:
            self._resident(sid)
            t = self.tables[sid]
            if len(t) > max_blocks:
                raise BMError(EINVAL, "table longer than max_blocks")
            tables.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[sid])
        return tables, lens


def slots(bm, sid, start: int, count: int):
    """Slots of tokens [start, start+count) of a sequence: token t lives in
    logical block t // B at offset t % B ("Pages, from operating systems")."""
    bm._resident(sid)
    if start < 0 or count < 0 or start + count > bm.lens[sid]:
        raise BMError(EINVAL, "tokens past the sequence's length")
    t = bm.tables[sid]
    return [t[i // bm.B] * bm.B + i % bm.B for i in range(start, start + count)]


def count_shared(bm, seq_ids) -> int:
    """Table entries of the listed sequences whose block is referenced by more
    than one table (a block shared through fork, "Pages, from operating
    systems"): the batch reads such a block once per sharer."""
    total = 0
    for sid in seq_ids:
        bm._resident(sid)
        total += sum(1 for b in bm.tables[sid] if bm.ref[b] > 1)
    return total


def run_ops(bm, ops):
    """Apply a request script (see workloads.script / random_script).  Returns
    the status code of every op, and the (slot, src, dst) of every append and
    the tuple of copy pairs of every swap, in op order."""
    codes, appends = [], []
    for op in ops:
        kind = op[0]
        try:
            if kind == "add":
                bm.add_seq(op[1], op[2])
            elif kind == "fork":
                bm.fork(op[1], op[2])
            elif kind == "append":
                appends.append(bm.append_slot(op[1]))
            elif kind == "extend":
                for _ in range(op[2]):
                    appends.append(bm.append_slot(op[1]))
            elif kind == "free":
                bm.free_seq(op[1])
            elif kind == "swap_out":
                appends.append(tuple(bm.swap_out(op[1])))
            elif kind == "swap_in":
                appends.append(tuple(bm.swap_in(op[1])))
            elif kind == "truncate_by":
                # cut op[2] tokens (more than the length is an invalid call)
                L = bm.lens.get(op[1], 0)
                bm.truncate(op[1], L - op[2])
            else:
                raise ValueError(kind)
            codes.append(OK)
        except BMError as e:
            codes.append(e.code)
    return codes, appends
