"""Continuous-batching decode loop for one attention layer on one GPU.

Drives the native scheduler (pkv_sched_*) and the device kernels step by step
(PagedAttention and Continuous Batching, "Batch by step, not by request";
PagedAttention: The vLLM Paper, "Continuous Batching" and "Implementation
Essentials"): every step

  1. the scheduler swaps preempted requests back in, hands out prefill chunks
     (continuing admitted requests first, within the optional per-step prefill
     budget), admits waiting requests into free blocks -- reusing cached blocks
     of their prompt's prefix when the request carries its token ids --,
     appends one slot per request whose prefill is complete (preempting the
     youngest when the pool runs dry: swapped to the host pool when the loop
     has one, else dropped for recomputation) and names the requests that
     finish;
  2. the swap-in copies (host to device), the swap-out copies (device to host)
     and the copy-on-write copies run, then one reshape_and_cache writes the
     KV of every prefill chunk;
  3. the multi-token attention kernel attends each chunk's rows causally over
     its sequence's cache, then paged decode attention runs over the batch's
     block tables (host work plan) and writes the new token of every decoding
     request into its slot as it goes;
  4. the finished requests give their blocks back.

The step's metadata (slots, block copy pairs, block tables, lengths, work plan)
is packed into one pinned host buffer and sent with a single asynchronous copy;
two buffers alternate so the host fills one while the previous step's copy may
still run.  The host pool, when there is one, is pinned host memory that the
swap kernel reads and writes over the host link.

K/V and query values come from caller-supplied sources (the loop computes no
model): kv_source(pairs) returns the K and V rows [T, Hkv, D] and
q_source(pairs) the query rows [T, Hq, D] for an int64 array of (request id,
token position) pairs.  Everything the method computes runs in libpkv.so.
With fp8 E4M3 pools (dtype torch.uint8) the rows stay bf16 and every call
takes the per-KV-head scales (kv_scales).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import (BlockManager, Plan, Scheduler, attention_plan, attention_workspace_bytes,
               copy_blocks, paged_attention_decode, paged_attention_prefill, pool_shapes,
               reshape_and_cache, swap_blocks)


def _pad4(n: int) -> int:
    return (n + 3) // 4 * 4   # int32 words to the next 16-byte boundary


class DecodeLoop:
    def __init__(self, *, num_blocks: int, block_size: int, q_heads: int, kv_heads: int,
                 head_dim: int, max_running: int, max_len: int, dtype=torch.bfloat16,
                 partition_size: int = 0, reserve_max: bool = False, free_order=None,
                 host_blocks: int = 0, max_prefill_tokens=None, kv_scales=None,
                 device="cuda"):
        self.B, self.Hq, self.Hkv, self.D = block_size, q_heads, kv_heads, head_dim
        self.P = partition_size
        self.max_len = max_len
        self.max_blocks = max(1, math.ceil(max_len / block_size))
        self.device = torch.device(device)
        self.fp8 = dtype == torch.uint8
        if self.fp8 != (kv_scales is not None):
            raise ValueError("fp8 pools (torch.uint8) go with kv_scales=(k_scale, v_scale)")
        self.k_scale, self.v_scale = kv_scales if self.fp8 else (None, None)
        self.bm = BlockManager(num_blocks, block_size, free_order)
        if host_blocks:
            self.bm.set_host_pool(host_blocks)
        self.sched = Scheduler(self.bm, max_running, reserve_max, swap=host_blocks > 0,
                               max_prefill_tokens=max_prefill_tokens)
        ks, vs = pool_shapes(num_blocks, kv_heads, head_dim, block_size, dtype)
        self.k_pool = torch.empty(ks, dtype=dtype, device=self.device)
        self.v_pool = torch.empty(vs, dtype=dtype, device=self.device)
        self.host_k = self.host_v = None
        if host_blocks:
            hks, hvs = pool_shapes(host_blocks, kv_heads, head_dim, block_size, dtype)
            self.host_k = torch.empty(hks, dtype=dtype, pin_memory=True)
            self.host_v = torch.empty(hvs, dtype=dtype, pin_memory=True)
        nbytes = attention_workspace_bytes(max_running, q_heads, head_dim, max_len,
                                           partition_size)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.device)
        self.out = torch.empty((max_running, q_heads, head_dim), dtype=torch.float32,
                               device=self.device)
        self._host = [None, None]      # pinned int32 staging buffers, used alternately
        self._done = [None, None]      # event after each buffer's last copy
        self._dev = None
        self._turn = 0

    def add_request(self, req_id: int, prompt_len: int, max_new_tokens: int,
                    tokens=None) -> None:
        """tokens: the prompt's token ids, or None (no prefix caching for it)."""
        if prompt_len + max_new_tokens > self.max_len:
            raise ValueError("request longer than the loop's max_len")
        self.sched.add_request(req_id, prompt_len, max_new_tokens, tokens=tokens)

    def _stage(self, parts):
        """Copy the int32 arrays `parts` (a dict) to the device in one transfer;
        returns device views of them by name (each on a 16-byte boundary)."""
        total = sum(_pad4(p.size) for p in parts.values())
        i = self._turn
        self._turn ^= 1
        if self._done[i] is not None:
            self._done[i].synchronize()    # its previous copy has left the buffer
        if self._host[i] is None or self._host[i].numel() < total:
            cap = max(total, 1 << 16) * 2
            self._host[i] = torch.empty(cap, dtype=torch.int32, pin_memory=True)
            if self._dev is None or self._dev.numel() < cap:
                self._dev = torch.empty(cap, dtype=torch.int32, device=self.device)
        host = self._host[i].numpy()
        off, spans = 0, {}
        for name, p in parts.items():
            host[off:off + p.size] = p.reshape(-1)
            spans[name] = (off, p.size)
            off += _pad4(p.size)
        self._dev[:total].copy_(self._host[i][:total], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self._done[i] = ev
        return {name: self._dev[o:o + n] for name, (o, n) in spans.items()}

    def step(self, kv_source, q_source):
        """One iteration.  Returns (the scheduler's step dict -- plus "stats",
        the scheduler's (tokens held, slots committed, waiting, running,
        swapped) taken before the finished requests leave --, the decode
        attention output [n_batch, Hq, D], the prefill attention output
        [prefill rows, Hq, D] for the step's chunks in order -- views valid
        until the next step -- and the host context lengths of the batch)."""
        st = self.sched.begin_step()
        ids = st["batch"]
        n = len(ids)
        chunks = st["prefill"]
        # token rows: the prefill chunks (written by reshape_and_cache), then one
        # token per decoding request (written by the attention launch)
        pairs, write_slots = [], []
        for rid, start, cnt in chunks:
            write_slots.append(self.bm.slots(rid, start, cnt))
            pairs.append(np.stack([np.full(cnt, rid, np.int64),
                                   np.arange(start, start + cnt, dtype=np.int64)], 1))
        n_pf = sum(c for _, _, c in chunks)
        parts = {}
        if write_slots:
            parts["slots"] = np.concatenate(write_slots).view(np.int32)
            pf_ids = [rid for rid, _, _ in chunks]
            pf_tables, _ = self.bm.fill_batch(pf_ids, self.max_blocks)
            pf_lens = np.array([start + cnt for _, start, cnt in chunks], np.int32)
            pf_width = max(1, -(-int(pf_lens.max()) // self.B))
            parts.update(pf_tables=np.ascontiguousarray(pf_tables[:, :pf_width]).reshape(-1),
                         pf_lens=pf_lens,
                         pf_start=np.concatenate([[0], np.cumsum([c for _, _, c in chunks])])
                         .astype(np.int32))
        lens = np.empty(0, np.int32)
        if n:
            tables, lens = self.bm.fill_batch(ids, self.max_blocks)
            mcl = int(lens.max())
            width = max(1, -(-mcl // self.B))          # the batch's widest table
            tables = np.ascontiguousarray(tables[:, :width])
            words, n_items, n_merge = attention_plan(lens, self.Hkv, self.B, width, mcl,
                                                     self.P)
            pairs.append(np.stack([np.asarray(ids, np.int64), lens.astype(np.int64) - 1], 1))
            parts.update(tables=tables.reshape(-1), lens=lens, plan=words)
        for key in ("swap_in", "swap_out", "cow"):
            if st[key]:
                parts[key] = np.asarray(st[key], np.int32)
        dev = self._stage(parts) if parts else {}
        # every launch of the step goes to the current stream, looked up once
        stream = torch.cuda.current_stream().cuda_stream
        # block copies in the scheduler's order: swap-ins, swap-outs, copy-on-write
        if "swap_in" in dev:
            swap_blocks(self.k_pool, self.v_pool, self.host_k, self.host_v,
                        dev["swap_in"].view(-1, 2), stream=stream)
        if "swap_out" in dev:
            swap_blocks(self.host_k, self.host_v, self.k_pool, self.v_pool,
                        dev["swap_out"].view(-1, 2), stream=stream)
        if "cow" in dev:
            copy_blocks(self.k_pool, self.v_pool, dev["cow"].view(-1, 2), stream=stream)
        out = self.out[:n]
        out_pf = None
        if pairs:
            all_pairs = np.concatenate(pairs)
            k, v = kv_source(all_pairs)
            q = q_source(all_pairs)
            if n_pf:
                reshape_and_cache(k[:n_pf], v[:n_pf], self.k_pool, self.v_pool,
                                  dev["slots"].view(torch.int64), stream=stream,
                                  k_scale=self.k_scale, v_scale=self.v_scale)
                out_pf = self._prefill_out(n_pf)
                paged_attention_prefill(out_pf, q[:n_pf], self.k_pool, self.v_pool,
                                        dev["pf_tables"].view(len(chunks), -1), dev["pf_lens"],
                                        dev["pf_start"], max(c for _, _, c in chunks),
                                        stream=stream, k_scale=self.k_scale,
                                        v_scale=self.v_scale)
        if n:
            paged_attention_decode(out, q[n_pf:], self.k_pool, self.v_pool,
                                   dev["tables"].view(n, -1), dev["lens"], mcl,
                                   partition_size=self.P, workspace=self.ws,
                                   plan=Plan(dev["plan"], n_items, n_merge), stream=stream,
                                   new_key=k[n_pf:], new_value=v[n_pf:],
                                   k_scale=self.k_scale, v_scale=self.v_scale)
        st["stats"] = self.sched.stats()   # before the finished requests leave
        self.sched.end_step()
        return st, out, out_pf, lens

    def _prefill_out(self, rows: int) -> torch.Tensor:
        if getattr(self, "_pf_out", None) is None or self._pf_out.shape[0] < rows:
            self._pf_out = torch.empty((max(rows, 1024), self.Hq, self.D), dtype=torch.float32,
                                       device=self.device)
        return self._pf_out[:rows]

    def stats(self):
        """(tokens held, slots committed, waiting, running, swapped out)."""
        return self.sched.stats()

    def idle(self) -> bool:
        _, _, nw, nr, ns = self.sched.stats()
        return nw == 0 and nr == 0 and ns == 0
