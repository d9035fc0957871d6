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

The step's metadata (slots, block copy pairs, block tables, lengths, work plan,
the K/V row list) is packed by the library (pkv_pack_step) into one pinned host
buffer and sent with a single asynchronous copy; two buffers alternate so the
host fills one while the previous step's copy may still run.  The host pool, when there is one, is pinned host memory that the
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

import ctypes

from . import (BlockManager, LoopConfig, LoopSource, LoopStepInfo, Plan, PkvError, Scheduler,
               StepPack, attention_workspace, copy_blocks, lib, paged_attention_decode,
               paged_attention_prefill, pool_shapes, reshape_and_cache, swap_blocks)
from . import _check, _dev, _dtype_code, _stream


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
        self.ws = attention_workspace(max_running, q_heads, head_dim, max_len, partition_size,
                                      device=self.device)
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

    def _pack(self, stream):
        """pkv_pack_step of the step begun into a pinned buffer (two alternate,
        so the host fills one while the previous step's copy may still run),
        then one asynchronous copy to the device.  Returns (layout, host
        int32 view, device int32 buffer)."""
        i = self._turn
        self._turn ^= 1
        if self._done[i] is not None:
            self._done[i].synchronize()    # its previous copy has left the buffer
        lay = StepPack()
        while True:
            buf = self._host[i]
            if buf is not None and self.sched.pack_step(self.max_blocks, self.Hkv, self.P,
                                                        buf.numpy(), lay):
                break
            cap = max(lay.total_words, 1 << 16) * 2
            self._host[i] = torch.empty(cap, dtype=torch.int32, pin_memory=True)
            if self._dev is None or self._dev.numel() < cap:
                self._dev = torch.empty(cap, dtype=torch.int32, device=self.device)
        total = lay.total_words
        if total:
            self._dev[:total].copy_(self._host[i][:total], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(stream)
            self._done[i] = ev
        return lay, self._host[i].numpy(), self._dev

    def step(self, kv_source, q_source):
        """One iteration.  Returns (the scheduler's step dict -- plus "stats",
        the scheduler's (tokens held, slots committed, waiting, running,
        swapped) taken before the finished requests leave --, the decode
        attention output [n_batch, Hq, D], the prefill attention output
        [prefill rows, Hq, D] for the step's chunks in order -- views valid
        until the next step -- and the host context lengths of the batch)."""
        # every copy and launch of the step goes to the current stream, looked up once
        ts = torch.cuda.current_stream()
        stream = ts.cuda_stream
        st = self.sched.begin_step()
        n = len(st["batch"])
        nc = len(st["prefill"])
        lay, host, dev = self._pack(ts)
        n_pf = lay.n_prefill_rows

        def d(off, words):
            return dev[off:off + words]

        # block copies in the scheduler's order: swap-ins, swap-outs, copy-on-write
        if st["swap_in"]:
            swap_blocks(self.k_pool, self.v_pool, self.host_k, self.host_v,
                        d(lay.swap_in_off, 2 * len(st["swap_in"])).view(-1, 2), stream=stream)
        if st["swap_out"]:
            swap_blocks(self.host_k, self.host_v, self.k_pool, self.v_pool,
                        d(lay.swap_out_off, 2 * len(st["swap_out"])).view(-1, 2), stream=stream)
        if st["cow"]:
            copy_blocks(self.k_pool, self.v_pool, d(lay.cow_off, 2 * len(st["cow"])).view(-1, 2),
                        stream=stream)
        out = self.out[:n]
        out_pf = None
        lens = host[lay.lens_off:lay.lens_off + n].copy()
        # token rows: the prefill chunks (written by reshape_and_cache), then one
        # token per decoding request (written by the attention launch)
        if n_pf + n:
            pairs = host[lay.pairs_off:lay.pairs_off + 4 * (n_pf + n)].view(np.int64)
            pairs = pairs.reshape(-1, 2).copy()
            k, v = kv_source(pairs)
            q = q_source(pairs)
            if n_pf:
                reshape_and_cache(k[:n_pf], v[:n_pf], self.k_pool, self.v_pool,
                                  d(lay.slots_off, 2 * n_pf).view(torch.int64), stream=stream,
                                  k_scale=self.k_scale, v_scale=self.v_scale)
                out_pf = self._prefill_out(n_pf)
                paged_attention_prefill(out_pf, q[:n_pf], self.k_pool, self.v_pool,
                                        d(lay.pf_tables_off, nc * lay.pf_width).view(nc, -1),
                                        d(lay.pf_lens_off, nc), d(lay.pf_start_off, nc + 1),
                                        lay.pf_max_rows, stream=stream, k_scale=self.k_scale,
                                        v_scale=self.v_scale)
        if n:
            plan = Plan(d(lay.plan_off, 4 * lay.n_items + lay.n_merge), lay.n_items, lay.n_merge)
            paged_attention_decode(out, q[n_pf:], self.k_pool, self.v_pool,
                                   d(lay.tables_off, n * lay.width).view(n, -1),
                                   d(lay.lens_off, n), lay.max_context,
                                   partition_size=self.P, workspace=self.ws, plan=plan,
                                   stream=stream, new_key=k[n_pf:], new_value=v[n_pf:],
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


class NativeLoop:
    """The same loop with the whole step in one native call (pkv_loop_step):
    scheduling, packing, the metadata copy and every launch run in libpkv.so,
    and Python only makes the call.  The step's query and K/V rows come from
    device banks (set_source): row r of the step, the token (request id,
    position), reads bank row (id * mul + position) mod bank rows.  Same
    arguments as DecodeLoop; step() returns the pkv_loop_step_info of the step
    (counts, stats, host_us / wait_us), outputs() copies the step's decode and
    prefill outputs into new tensors."""

    def __init__(self, *, num_blocks: int, block_size: int, q_heads: int, kv_heads: int,
                 head_dim: int, max_running: int, max_len: int, dtype=torch.bfloat16,
                 partition_size: int = 0, reserve_max: bool = False, free_order=None,
                 host_blocks: int = 0, max_prefill_tokens=None, kv_scales=None,
                 device="cuda", stream=None):
        self.B, self.Hq, self.Hkv, self.D = block_size, q_heads, kv_heads, head_dim
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
        self.stream = _stream(stream)
        cfg = LoopConfig(num_blocks, block_size, q_heads, kv_heads, head_dim, max_running, max_len,
                         partition_size, host_blocks, _dtype_code(self.k_pool))
        h = ctypes.c_void_p()
        scales = (_dev(self.k_scale, "k_scale"), _dev(self.v_scale, "v_scale")) if self.fp8 \
            else (None, None)
        hosts = (self.host_k.data_ptr(), self.host_v.data_ptr()) if host_blocks else (None, None)
        _check(lib.pkv_loop_create(ctypes.byref(cfg), self.bm._h, self.sched._h,
                                   _dev(self.k_pool, "k_pool"), _dev(self.v_pool, "v_pool"),
                                   *hosts, *scales, self.stream, ctypes.byref(h)),
               "pkv_loop_create")
        self._h = h
        self._src = None
        self._info = LoopStepInfo()

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib.pkv_loop_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_request(self, req_id: int, prompt_len: int, max_new_tokens: int,
                    tokens=None) -> None:
        self.sched.add_request(req_id, prompt_len, max_new_tokens, tokens=tokens)

    def set_source(self, q_bank: torch.Tensor, k_bank: torch.Tensor, v_bank: torch.Tensor,
                   q_mul: int, kv_mul: int) -> None:
        """q_bank bf16 [rows, Hq, D], k_bank / v_bank bf16 [rows, Hkv, D] (device)."""
        rows = q_bank.shape[0]
        for t, heads, name in ((q_bank, self.Hq, "q_bank"), (k_bank, self.Hkv, "k_bank"),
                               (v_bank, self.Hkv, "v_bank")):
            if t.dtype != torch.bfloat16 or tuple(t.shape) != (rows, heads, self.D) or \
                    not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous bf16 [rows, heads, D]")
        self._banks = (q_bank, k_bank, v_bank)
        self._src = LoopSource(_dev(q_bank, "q_bank"), _dev(k_bank, "k_bank"),
                               _dev(v_bank, "v_bank"), rows, int(q_mul), int(kv_mul))

    def step(self) -> LoopStepInfo:
        if self._src is None:
            raise ValueError("set_source first")
        code = lib.pkv_loop_step(self._h, ctypes.byref(self._src), ctypes.byref(self._info))
        if code != 0:
            raise PkvError(code, "pkv_loop_step")
        return self._info

    def outputs(self):
        """The last step's decode output [n_batch, Hq, D] and prefill output
        [n_prefill_rows, Hq, D] (float32 copies)."""
        info = self._info
        dec = torch.empty((info.n_batch, self.Hq, self.D), dtype=torch.float32, device=self.device)
        pf = torch.empty((info.n_prefill_rows, self.Hq, self.D), dtype=torch.float32,
                         device=self.device)
        _check(lib.pkv_loop_copy_outputs(self._h, dec.data_ptr() if info.n_batch else None,
                                         pf.data_ptr() if info.n_prefill_rows else None),
               "pkv_loop_copy_outputs")
        return dec, pf

    def stats(self):
        return self.sched.stats()

    def idle(self) -> bool:
        _, _, nw, nr, ns = self.sched.stats()
        return nw == 0 and nr == 0 and ns == 0
