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

    # -- queries -------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, block: int) -> int:
        if not 0 <= block < self.N:
            raise BMError(EINVAL, "block out of range")
        return self.ref[block]

    def seq_info(self, sid: int):
        if sid not in self.tables:
            raise BMError(ENOSEQ)
        return self.lens[sid], len(self.tables[sid])

    def block_table(self, sid: int):
        if sid not in self.tables:
            raise BMError(ENOSEQ)
        return list(self.tables[sid])

    def snapshot(self):
        return list(self.ref), list(self.free)

    # -- updates -------------------------------------------------------------
    def _take(self) -> int:
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def add_seq(self, sid: int, num_tokens: int) -> None:
        if num_tokens < 0:
            raise BMError(EINVAL, "negative length")
        if sid in self.tables:
            raise BMError(EEXIST)
        need = -(-num_tokens // self.B)
        if need > len(self.free):
            raise BMError(ENOBLOCKS)
        self.tables[sid] = [self._take() for _ in range(need)]
        self.lens[sid] = num_tokens

    def append_slot(self, sid: int):
        """Reserve the slot for the sequence's next token.  Returns
        (slot, cow_src, cow_dst); cow_src = cow_dst = -1 when no copy is due."""
        if sid not in self.tables:
            raise BMError(ENOSEQ)
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
        if parent not in self.tables:
            raise BMError(ENOSEQ)
        if child in self.tables:
            raise BMError(EEXIST)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, sid: int) -> None:
        if sid not in self.tables:
            raise BMError(ENOSEQ)
        for b in self.tables.pop(sid):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[sid]

    def fill_batch(self, sids, max_blocks: int):
        """Block tables [n, max_blocks] (padded with -1) and context lengths."""
        tables, lens = [], []
        for sid in sids:
            if sid not in self.tables:
                raise BMError(ENOSEQ)
            t = self.tables[sid]
            if len(t) > max_blocks:
                raise BMError(EINVAL, "table longer than max_blocks")
            tables.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[sid])
        return tables, lens


def slots(bm, sid, start: int, count: int):
    """Slots of tokens [start, start+count) of a sequence: token t lives in
    logical block t // B at offset t % B ("Pages, from operating systems")."""
    if sid not in bm.tables:
        raise BMError(ENOSEQ)
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
        if sid not in bm.tables:
            raise BMError(ENOSEQ)
        total += sum(1 for b in bm.tables[sid] if bm.ref[b] > 1)
    return total


def run_ops(bm, ops):
    """Apply a request script (see workloads.script / random_script).  Returns
    the status code of every op and the (slot, src, dst) of every append."""
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
            else:
                raise ValueError(kind)
            codes.append(OK)
        except BMError as e:
            codes.append(e.code)
    return codes, appends
