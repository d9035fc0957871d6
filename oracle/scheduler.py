"""Reference iteration-level (continuous) batching scheduler -- TEST
INFRASTRUCTURE ONLY (plain Python over the reference block manager; the product
never imports it).

From the pages:
  * scheduling works at the level of single decoding iterations: after every
    step, finished sequences leave the batch and waiting ones join ("PagedAttention
    and Continuous Batching", "Batch by step, not by request"; "PagedAttention:
    The vLLM Paper", "Continuous Batching: Request-Level vs. Iteration-Level
    Scheduling", whose figure has A finish, A dequeue and D enqueue, giving the
    batch {B, C, D});
  * with paging a new request only needs free blocks, not a large contiguous
    region (same section of the first page);
  * under memory pressure a running request is preempted: its blocks are swapped
    to CPU memory, or dropped and its KV recomputed later ("Implementation
    Essentials", block manager; OS-paging analogy table, "Swapping");
  * the systems before paging reserved a region per request for its maximum
    length ("Background and Motivation").

Readings where the pages are silent:
  * requests are admitted first-come first-served: admission stops at the first
    waiting request that does not fit (no skipping ahead) and at most
    `max_running` requests run at once;
  * paged policy: admitting a request allocates blocks for its current context
    (its prompt plus the tokens it generated before any preemption);
  * reserve policy (the max-length reservation of the earlier systems,
    simulated over the same pool): a request is admitted only if the blocks not
    yet reserved cover its maximum length ceil((prompt + max_new) / B); they stay
    reserved until it finishes, so its appends can never run out of blocks;
  * every running request (one admitted this step included) produces one token
    per step, and the running requests append their slots in admission order;
  * when an append finds no free block (paged policy), the most recently
    admitted running request is preempted: its blocks are freed, it returns to
    the FRONT of the waiting queue keeping the tokens it generated (they are
    rebuilt with its prompt on re-admission), and the append is retried;
  * a request finishes in the step that produces its max_new-th token and is
    freed by end_step(), after the step's batch tables have been read;
  * a request whose maximum length can never fit the pool is rejected when it
    is submitted;
  * begin_step() and end_step() alternate; calling either out of turn is an
    error.

Swap policy (swap=True, over a block manager with a host pool):
  * the preempted request's blocks move to the host (block manager swap_out)
    when the host has a block for each of them; otherwise it is dropped and
    recomputed as above.  A request admitted in the same step holds no KV yet
    (its prefill is written after scheduling), so it is always dropped;
  * swapped requests wait in their own queue, the most recently preempted
    behind the others as for dropped ones (each victim goes to the front);
  * each step first swaps requests back in from the front of that queue while
    fewer than max_running run and the device has a block for each of their
    blocks (no skipping ahead); a resumed request rejoins the running list at
    its end, keeping its tokens;
  * no waiting request is admitted while any request is still swapped out;
  * the caller runs a step's copies in this order: swap-ins (host to device),
    swap-outs (device to host: they may reuse host blocks the swap-ins just
    released), copy-on-write copies, prefill writes, then the token writes and
    attention.

Prefix caching and chunked prefill ("Impact and Follow-Ups": a cached prompt
prefix makes that part of the prefill free; long prompts are split into chunks
interleaved with decode):
  * a request may carry its prompt's token ids; it is then admitted with the
    block manager's add_seq_prefix, and the tokens already cached are not
    prefilled again (a request admitted again after being dropped finds its
    prompt blocks the same way; its generated tokens are always recomputed);
  * with a prefill budget of C tokens per step, each step first continues the
    prefills of admitted requests in admission order, then admits new requests
    while budget is left; each gets a chunk of at most the budget left.  No
    budget (None) means every prefill completes in its admission step;
  * a request produces a token only in steps where its prefill is complete,
    including the step its last chunk runs in; the batch lists the requests
    that produced a token;
  * a chunk's full prompt blocks join the prefix cache when the chunk is
    issued (the caller writes every chunk of a step before anything reads
    them; a request admitted later in the same step may already reuse them);
  * a preempted request's chunk of the same step is undone (its KV for that
    chunk is never written) and its cache entries for it are withdrawn, so a
    swapped request resumes its prefill where its written KV ends.  The
    youngest request is preempted first, so any request that reused those
    blocks in the same step is preempted before them.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass

from oracle.block_manager import BMError, EEXIST, EINVAL, ENOBLOCKS


@dataclass
class Request:
    rid: int
    prompt: int
    max_new: int
    generated: int = 0
    reserved: int = 0   # blocks held by a reservation (reserve policy)
    tokens: list | None = None   # prompt token ids, when known
    target: int = 0     # context to prefill since the last admission
    prefilled: int = 0  # tokens of it whose KV is written (or cached)

    @property
    def ctx(self) -> int:
        """Tokens whose KV the request holds (or must rebuild) right now."""
        return self.prompt + self.generated


class Scheduler:
    def __init__(self, bm, max_running: int, reserve_max: bool = False, swap: bool = False,
                 max_prefill_tokens: int | None = None):
        if max_running <= 0:
            raise BMError(EINVAL, "max_running must be positive")
        if max_prefill_tokens is not None and max_prefill_tokens <= 0:
            raise BMError(EINVAL, "the prefill budget must be positive")
        if reserve_max and swap:
            raise BMError(EINVAL, "the reserve policy never preempts")
        self.bm = bm
        self.max_running = max_running
        self.reserve_max = reserve_max
        self.swap = swap
        self.max_prefill = max_prefill_tokens
        self.swapped: deque[Request] = deque()
        self.waiting: deque[Request] = deque()
        self.running: list[Request] = []
        self.known: set[int] = set()
        self.reserved = 0
        self.finishing: list[Request] = []
        self.in_step = False

    def _blocks(self, tokens: int) -> int:
        return -(-tokens // self.bm.B)

    def add_request(self, rid: int, prompt: int, max_new: int, tokens=None) -> None:
        if prompt < 0 or max_new < 1:
            raise BMError(EINVAL, "prompt must be >= 0 and max_new >= 1")
        if tokens is not None and len(tokens) != prompt:
            raise BMError(EINVAL, "token ids must cover the prompt")
        if rid in self.known:
            raise BMError(EEXIST)
        if self._blocks(prompt + max_new) > self.bm.N:
            raise BMError(EINVAL, "request can never fit the pool")
        self.known.add(rid)
        self.waiting.append(Request(rid, prompt, max_new,
                                    tokens=None if tokens is None else [int(t) for t in tokens]))

    def begin_step(self):
        """One iteration: swap-ins, prefill chunks and admissions, then one
        slot per request whose prefill is complete.  Returns dict(batch (the
        requests that produced a token), slots, cow, admitted=[(rid, ctx,
        cached)], prefill=[(rid, start, n)], preempted (dropped), finished,
        swap_in=[(host, device)], swap_out=[(device, host)], swapped_in,
        swapped_out)."""
        if self.in_step:
            raise BMError(EINVAL, "end_step() was not called")
        self.in_step = True
        swap_in, swapped_in = [], []
        while self.swapped and len(self.running) < self.max_running:
            r = self.swapped[0]
            try:
                swap_in += self.bm.swap_in(r.rid)
            except BMError as e:
                if e.code == ENOBLOCKS:
                    break
                raise
            self.swapped.popleft()
            self.running.append(r)
            swapped_in.append(r.rid)

        # prefill chunks: admitted requests first, in admission order
        budget = float("inf") if self.max_prefill is None else self.max_prefill
        chunks: list[list] = []                     # [request, start, n]

        def give_chunk(r):
            nonlocal budget
            n = int(min(r.target - r.prefilled, budget))
            if n > 0:
                chunks.append([r, r.prefilled, n])
                r.prefilled += n
                budget -= n
                if r.tokens is not None:        # the chunk's full blocks join the cache
                    self.bm.register_prefix(r.rid, r.tokens, r.prefilled)

        for r in self.running:
            if r.prefilled < r.target and budget > 0:
                give_chunk(r)

        admitted: list[tuple[Request, int, int]] = []   # (request, context, cached)
        while self._may_admit() and self.waiting and len(self.running) < self.max_running \
                and budget > 0:
            r = self.waiting[0]
            need_max = self._blocks(r.prompt + r.max_new)
            if self.reserve_max and self.reserved + need_max > self.bm.N:
                break
            try:
                if r.tokens is not None:
                    cached = self.bm.add_seq_prefix(r.rid, r.tokens, r.ctx)
                else:
                    self.bm.add_seq(r.rid, r.ctx)
                    cached = 0
            except BMError as e:
                if e.code == ENOBLOCKS:
                    break
                raise
            if self.reserve_max:
                r.reserved = need_max
                self.reserved += need_max
            self.waiting.popleft()
            self.running.append(r)
            r.target, r.prefilled = r.ctx, cached
            admitted.append((r, r.ctx, cached))
            give_chunk(r)

        slots, cow, preempted, swap_out, swapped_out = [], [], [], [], []
        decoding: list[Request] = []
        i = 0
        while i < len(self.running):
            r = self.running[i]
            if r.prefilled < r.target:              # still prefilling: no token this step
                i += 1
                continue
            try:
                slot, src, dst = self.bm.append_slot(r.rid)
            except BMError as e:
                if e.code != ENOBLOCKS:
                    raise
                victim = self._victim()
                fresh = any(a is victim for a, _, _ in admitted)
                for ch in chunks:                   # its chunk of this step is not written
                    if ch[0] is victim:
                        victim.prefilled -= ch[2]
                        chunks.remove(ch)
                        self.bm.unregister_prefix(victim.rid, victim.prefilled)
                        break
                if self._swap_victim(victim, fresh):
                    swap_out += self.bm.swap_out(victim.rid)
                    swapped_out.append(victim.rid)
                    self.swapped.appendleft(victim)
                    continue
                self.bm.free_seq(victim.rid)
                admitted = [a for a in admitted if a[0] is not victim]
                preempted.append(victim.rid)
                self.waiting.appendleft(victim)
                continue
            slots.append(slot)
            if src >= 0:
                cow.append((src, dst))
            decoding.append(r)
            i += 1

        finished = []
        for r in decoding:
            r.generated += 1
            if r.generated == r.max_new:
                finished.append(r.rid)
                self.finishing.append(r)
        return {
            "batch": [r.rid for r in decoding],
            "slots": slots,
            "cow": cow,
            "admitted": [(r.rid, n, c) for r, n, c in admitted],
            "prefill": [(r.rid, start, n) for r, start, n in chunks],
            "preempted": preempted,
            "finished": finished,
            "swap_in": swap_in,
            "swap_out": swap_out,
            "swapped_in": swapped_in,
            "swapped_out": swapped_out,
        }

    # -- policy decisions ----------------------------------------------------------
    def _victim(self) -> Request:
        """The preempted request: the most recently admitted one."""
        return self.running.pop()

    def _may_admit(self) -> bool:
        """New requests wait while any preempted one is still swapped out."""
        return not self.swapped

    def _swap_victim(self, victim: Request, fresh: bool) -> bool:
        """Swap (rather than drop) a victim that holds KV, when the host has a
        block for each of its blocks."""
        return self.swap and not fresh and \
            self.bm.seq_info(victim.rid)[1] <= self.bm.num_free_host()

    def end_step(self) -> None:
        """Free the requests that finished in the step."""
        if not self.in_step:
            raise BMError(EINVAL, "no step in progress")
        self.in_step = False
        for r in self.finishing:
            self.bm.free_seq(r.rid)
            self.running.remove(r)
            self.reserved -= r.reserved
        self.finishing = []

    # -- accounting ------------------------------------------------------------
    def tokens_held(self) -> int:
        return sum(r.ctx for r in self.running)

    def slots_committed(self) -> int:
        """Slots the policy keeps for the running requests: allocated blocks
        (paged) or reserved blocks (reserve policy), times B."""
        if self.reserve_max:
            return self.reserved * self.bm.B
        return (self.bm.N - self.bm.num_free()) * self.bm.B

    def idle(self) -> bool:
        return not self.waiting and not self.running and not self.swapped
