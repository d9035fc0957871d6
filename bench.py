#!/usr/bin/env python3
"""Decode-step benchmark of the PagedAttention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

One step is one pass of the whole device path over one batch that already sits
in HBM: copy-on-write block copies (when the batch has any), the write of the
step's new tokens into their slots, the paged-attention main kernel and the
log-sum-exp reduce, for one attention layer.  When every sequence appends one
token at its last position (a decode step) the main kernel writes the tokens
itself; otherwise, or with --separate-cache-write, reshape_and_cache runs
first.  The host block manager builds
the batch (slots, copy pairs, block tables) once before timing; its cost is
reported separately.

As in a model, every layer has its own K/V pool while all layers share the
block tables; consecutive steps take consecutive layers, and there are enough
layers that at least 4 GiB of pool lies between two visits of one layer.  So a
step never finds the previous step's KV in the 256 MB last-level cache.

Prints ONE JSON line.  `value` is KV-read GB/s over the whole step: the
algorithmic KV bytes of the batch (valid tokens only, sum_s L_s * Hkv * D * 2 *
sizeof(kv)) times K, divided by the wall time of the K timed steps.  The
`roofline` object gives the main attention kernel's own rate (the same bytes
over its average launch time from HIP events on its stream, recorded around
the launch of every 8th timed step) against the HBM peak.  `also` holds the
same figures for the 70B-shaped long-context batch at both block sizes,
measured in the same run by child processes of this script (--no-extra skips
them).  `cpu_baseline` times the
fp64 CPU oracle's whole step on the same batch.

Inputs are synthetic (seeded), shaped like the pages' workloads; see
workloads/__init__.py for the recipe.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn decode KV-read GB/s (% of HBM peak) and decode tokens/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD's published figure
HOST_LINK_PEAK_GBS = 64.0      # PCIe 5.0 x16 host link, per direction, before protocol overhead
# the main kernel's source and the device headers it includes
MAIN_KERNEL_SRCS = [os.path.join(ROOT, "paged_kv_cache_346_amd", "csrc", n)
                    for n in ("attention.hip", "device_common.h", "kv_tiles.h", "decode_config.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MERGE_IN_LAUNCH_MAX = 16       # partitions per sequence the main launch merges itself
EVENT_EVERY = 8                # timed steps per main-kernel launch bracketed by events

DESCRIPTIONS = {
    "tiny_mha_f32": "tiny MHA decode: 4 seqs, 4 heads, D 64, B 16, fp32, L {1,15,16,70}, "
                    "+ 4 new tokens, one per sequence",
    "opt13b_mha": "OPT-13B-shaped layer decode: 64 seqs, 40 heads (MHA), D 128, B 16, bf16 KV, "
                  "L uniform [128,2048]",
    "llama8b_gqa": "Llama-3-8B-shaped GQA decode: 256 seqs, 32 q heads / 8 KV heads, D 128, "
                   "B 16, bf16 KV, L log-normal (median 600, sigma 0.8) clipped [16,4096], "
                   "+ 256 new tokens, one per sequence",
    "sampling_steady": "parallel sampling, steady step: 32 prompts x 8 samples, 1024-token "
                       "shared prompt blocks (refcount 8), 32/8 heads, D 128, B 16, bf16",
    "sampling_fork": "parallel sampling, fork step: 32 prompts x 8 samples, 224 copy-on-write "
                     "block copies before the token writes, 32/8 heads, D 128, B 16, bf16",
    "long70b_b16": "70B-shaped long-context decode: 16 seqs x 32768 tokens, 64 q heads / 8 KV "
                   "heads, D 128, B 16, bf16, 512-token partitions + log-sum-exp reduce",
    "long70b_b32": "70B-shaped long-context decode: 16 seqs x 32768 tokens, 64 q heads / 8 KV "
                   "heads, D 128, B 32, bf16, 512-token partitions + log-sum-exp reduce",
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    for path in MAIN_KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, launches_per_step: int):
    """HBM bytes per main-kernel launch from the committed counter summary, or
    None when there is none for this workload or the kernel source changed
    since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


class Batch:
    """One decode batch, built through the product's block manager and resident
    on the device."""

    def __init__(self, pkv, torch, W, name: str, partition_size=None, layers=0, use_plan=True,
                 append=True, kv_dtype=None):
        import numpy as np
        self.cfg = c = W.CONFIGS[name]
        self.kv_dtype = kv_dtype or c.dtype
        self.fp8 = self.kv_dtype == "fp8"
        if self.kv_dtype not in (c.dtype, "fp8") or (self.fp8 and c.dtype != "bf16"):
            raise ValueError(f"{name} is a {c.dtype} workload; fp8 KV goes with bf16 "
                             f"workloads only")
        self.w = w = W.make(name, pools=False)
        t0 = time.perf_counter()
        bm = pkv.BlockManager(w.num_blocks, c.B, w.free_order)
        for op in w.ops:
            if op[0] == "add":
                bm.add_seq(op[1], op[2])
            elif op[0] == "fork":
                bm.fork(op[1], op[2])
            elif op[0] == "extend":
                for _ in range(op[2]):
                    bm.append_slot(op[1])
        self.setup_s = time.perf_counter() - t0
        self.max_blocks = max(1, max(-(-int(L) // c.B) for L in w.lengths))
        ids = list(range(c.S))
        # the step's host bookkeeping: one append per running sequence + batch tables
        t0 = time.perf_counter()
        if w.step_ids:
            slots, pairs = bm.append_slots(w.step_ids)
        else:
            slots, pairs = None, None
        tables, lens = bm.fill_batch(ids, self.max_blocks)
        self.host_bookkeeping_us = (time.perf_counter() - t0) * 1e6
        assert lens.tolist() == w.lengths.tolist()
        self.bm = bm
        self.tables_host, self.lens_host = tables, lens

        dev = torch.device("cuda")
        tdt = torch.float32 if c.dtype == "f32" else torch.bfloat16
        ks, vs = pkv.pool_shapes(w.num_blocks, c.Hkv, c.D, c.B, tdt)
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 + c.seed)

        def normal(shape):
            x = torch.empty(shape, dtype=tdt, device=dev)
            flat = x.view(-1)
            chunk = 1 << 28
            for lo in range(0, flat.numel(), chunk):
                hi = min(flat.numel(), lo + chunk)
                flat[lo:hi] = torch.randn(hi - lo, generator=gen, device=dev,
                                          dtype=torch.float32).to(tdt)
            return x

        def codes(shape):
            # finite E4M3 codes of magnitude below 4 (exponent field < 10), random sign
            mag = torch.randint(0, 0x50, shape, generator=gen, device=dev, dtype=torch.uint8)
            sign = torch.randint(0, 2, shape, generator=gen, device=dev, dtype=torch.uint8)
            return mag | (sign << 7)

        esize = 4 if c.dtype == "f32" else 1 if self.fp8 else 2
        pool_bytes = 2 * w.num_blocks * c.Hkv * c.D * c.B * esize
        self.layers = layers or max(2, min(16, -(-(4 << 30) // pool_bytes)))
        if self.fp8:
            ks, vs = pkv.pool_shapes(w.num_blocks, c.Hkv, c.D, c.B, torch.uint8)
            self.pools = [(codes(ks), codes(vs)) for _ in range(self.layers)]
            # per-KV-head scales in the range a calibration would give for unit-variance K/V
            self.k_scale = torch.linspace(0.02, 0.03, c.Hkv, device=dev, dtype=torch.float32)
            self.v_scale = torch.linspace(0.03, 0.02, c.Hkv, device=dev, dtype=torch.float32)
        else:
            self.pools = [(normal(ks), normal(vs)) for _ in range(self.layers)]
            self.k_scale = self.v_scale = None
        self.pool_bytes = pool_bytes
        self.k_pool, self.v_pool = self.pools[0]
        self.q = self._to_dev(torch, w.q)
        self.slots = None if slots is None else torch.from_numpy(slots).to(dev)
        # a decode step appends one token per sequence, in batch order: the
        # attention launch can write them itself
        self.append = bool(append and slots is not None and list(w.step_ids) == ids)
        self.k_new = self._to_dev(torch, w.k_new) if slots is not None else None
        self.v_new = self._to_dev(torch, w.v_new) if slots is not None else None
        self.pairs = (torch.from_numpy(pairs).to(dev)
                      if pairs is not None and len(pairs) else None)
        self.n_pairs = 0 if self.pairs is None else int(self.pairs.shape[0])
        self.tables = torch.from_numpy(tables).to(dev)
        self.lens = torch.from_numpy(lens).to(dev)
        self.mcl = int(lens.max())
        self.P = c.partition_size if partition_size is None else partition_size
        self.ws = pkv.attention_workspace(c.S, c.Hq, c.D, self.mcl, self.P, device=dev)
        self.out = torch.empty((c.S, c.Hq, c.D), dtype=torch.float32, device=dev)
        self.kv_bytes = w.kv_bytes // 2 if self.fp8 else w.kv_bytes
        self.kv_elem_bytes = esize
        # blocks shared by several sequences are read with cached loads
        self.shared_entries = bm.count_shared(ids)
        self.shared_kv = self.shared_entries > 0
        # host work plan: exactly the batch's work items, largest first
        self.plan = None
        if use_plan:
            t0 = time.perf_counter()
            words, n_items, n_merge = pkv.attention_plan(lens, c.Hkv, c.B, self.max_blocks,
                                                         self.mcl, self.P)
            self.host_plan_us = (time.perf_counter() - t0) * 1e6
            dev_words = torch.from_numpy(words if words.size else np.zeros(4, np.int32)).to(dev)
            self.plan = pkv.Plan(dev_words, n_items, n_merge)
        torch.cuda.synchronize()

    @staticmethod
    def _to_dev(torch, a):
        import numpy as np
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    def step(self, pkv, layer=0, ev=None, main_ev=None):
        """Launch one step on `layer`'s pools.  `ev` (5 events) brackets
        copy_blocks, reshape_and_cache, the attention main kernel and the reduce;
        `main_ev` (2 events) brackets the main kernel only."""
        self.k_pool, self.v_pool = self.pools[layer % self.layers]
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        if self.pairs is not None:
            pkv.copy_blocks(self.k_pool, self.v_pool, self.pairs)
        rec(1)
        if self.slots is not None and not self.append:
            pkv.reshape_and_cache(self.k_new, self.v_new, self.k_pool, self.v_pool, self.slots,
                                  k_scale=self.k_scale, v_scale=self.v_scale)
        rec(2)
        if main_ev is not None:
            main_ev[0].record()
        nk, nv = (self.k_new, self.v_new) if self.append else (None, None)
        pkv.paged_attention_main(self.out, self.q, self.k_pool, self.v_pool, self.tables,
                                 self.lens, self.mcl, partition_size=self.P, workspace=self.ws,
                                 shared_kv=self.shared_kv, plan=self.plan, new_key=nk,
                                 new_value=nv, k_scale=self.k_scale, v_scale=self.v_scale)
        if main_ev is not None:
            main_ev[1].record()
        rec(3)
        pkv.paged_attention_reduce(self.out, self.lens, self.cfg.Hkv, self.cfg.B, self.max_blocks,
                                   self.mcl, partition_size=self.P, workspace=self.ws,
                                   plan=self.plan)
        rec(4)

    def launches(self):
        """Which of the four step kernels this batch launches (the reduce only
        when some sequence has more partitions than the main launch merges
        itself)."""
        nparts = -(-self.mcl // (self.P or 512))
        in_launch = nparts <= MERGE_IN_LAUNCH_MAX and self.cfg.S * self.cfg.Hkv <= 16384
        return (self.pairs is not None, self.slots is not None and not self.append, True,
                nparts > 1 and not in_launch)


def cpu_share() -> int:
    """Host cores this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when that is set."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(omp))) if omp.isdigit() and int(omp) > 0 else n


def cpu_baseline(batch, torch, budget_s: float):
    """The fp64 oracle's whole decode step on the same batch -- the step's
    token writes into the pools (oracle.cache_ops.reshape_and_cache), then
    attention of every (sequence, query head) through the block tables
    (oracle.attention.paged_attention_decode) -- repeated until about
    `budget_s` seconds (at least once), with BLAS threads = the process's CPU
    share; returns the JSON object."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle.attention import paged_attention_decode as oracle_decode
    from oracle.cache_ops import reshape_and_cache as oracle_cache

    c = batch.cfg

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    kp, vp, q = host(batch.k_pool), host(batch.v_pool), host(batch.q)
    scales = {}
    if batch.fp8:
        scales = {"k_scale": batch.k_scale.cpu().numpy(), "v_scale": batch.v_scale.cpu().numpy()}
    writes = batch.slots is not None
    if writes:
        slots = batch.slots.cpu().numpy()
        k_new, v_new = host(batch.k_new), host(batch.v_new)
    cores = cpu_share()
    elapsed, passes = 0.0, 0
    with threadpool_limits(limits=cores):
        while passes == 0 or (elapsed < budget_s and passes < 50):
            t0 = time.perf_counter()
            kq, vq = kp, vp
            if writes:
                kq, vq = oracle_cache(kp, vp, k_new, v_new, slots, **scales)
            oracle_decode(q, kq, vq, batch.tables_host, batch.lens_host, **scales)
            elapsed += time.perf_counter() - t0
            passes += 1
    kv = batch.kv_bytes * passes
    return {
        "value": round(kv / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"fp64 oracle decode step of the whole batch ({c.S} sequences, all {c.Hq} "
                  f"query heads): " + (f"the step's {len(slots)} token writes into the pools, "
                                       if writes else "") +
                  f"then gather through the block table + softmax(qK^T*scale)V; {passes} "
                  f"step(s), {kv / 1e6:.1f} MB of KV, {elapsed:.1f} s; BLAS threads = {cores}",
        "seconds": round(elapsed, 3),
        "steps": passes,
        "tokens_per_s": round(c.S * passes / elapsed, 4),
    }


def _swap_probe(torch, pkv, Hkv, D, B, N, n_blocks=2048, reps=5):
    """swap_blocks bandwidth over the host link: n_blocks random device blocks
    to a pinned host pool and back, timed with HIP events on the launch
    stream, best of `reps`."""
    dev = torch.device("cuda")
    ks, vs = pkv.pool_shapes(N, Hkv, D, B, torch.bfloat16)
    hks, hvs = pkv.pool_shapes(n_blocks, Hkv, D, B, torch.bfloat16)
    k = torch.zeros(ks, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(vs, dtype=torch.bfloat16, device=dev)
    hk = torch.zeros(hks, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.zeros(hvs, dtype=torch.bfloat16, pin_memory=True)
    g = torch.Generator().manual_seed(5)
    src = torch.randperm(N, generator=g)[:n_blocks].to(torch.int32)
    out_pairs = torch.stack([src, torch.arange(n_blocks, dtype=torch.int32)], 1).to(dev)
    in_pairs = torch.stack([torch.arange(n_blocks, dtype=torch.int32), src], 1).to(dev)
    nbytes = 2 * n_blocks * Hkv * D * B * 2
    res = {}
    for name, call in (("device_to_host", lambda: pkv.swap_blocks(hk, hv, k, v, out_pairs)),
                       ("host_to_device", lambda: pkv.swap_blocks(k, v, hk, hv, in_pairs))):
        call()
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            b.synchronize()
            best = min(best, a.elapsed_time(b) * 1e-3)
        res[name + "_GBps"] = round(nbytes / best / 1e9, 1)
    res.update(bytes_per_call=nbytes, blocks=n_blocks,
               link_peak_GBps_per_direction=HOST_LINK_PEAK_GBS)
    return res


class _PinnedIndex:
    """Device copies of host row indices through a ring of pinned buffers, so a
    synthetic K/V or query source never waits for the GPU: a copy from pageable
    memory would synchronise the stream, and with it host and device, every
    step."""

    def __init__(self, torch, dev, slots=4, cap=1 << 16):
        self.torch, self.dev = torch, dev
        self.bufs = [torch.empty(cap, dtype=torch.int64, pin_memory=True) for _ in range(slots)]
        self.done = [None] * slots
        self.i = 0
        self.stream = torch.cuda.current_stream()

    def __call__(self, idx):
        torch = self.torch
        i = self.i
        self.i = (i + 1) % len(self.bufs)
        if self.done[i] is not None:
            self.done[i].synchronize()       # the buffer's previous copy has left it
        n = idx.shape[0]
        if n > self.bufs[i].numel():
            self.bufs[i] = torch.empty(2 * n, dtype=torch.int64, pin_memory=True)
        self.bufs[i][:n].numpy()[:] = idx
        out = self.bufs[i][:n].to(self.dev, non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(self.stream)
        self.done[i] = ev
        return out


def run_serve(args, torch, np):
    """Continuous-batching loop over a synthetic request trace on the same pool
    (the Llama-3-8B-shaped layer's 16,162 blocks) under three policies: paged
    with preemption by dropping and recomputing, paged with preemption by
    swapping to a host pool of as many blocks, and the simulated max-length
    reservation of the earlier systems.  Also times swap_blocks over the host
    link.  Prints one JSON line (not the headline metric)."""
    import paged_kv_cache_346_amd as pkv
    from paged_kv_cache_346_amd.serve import DecodeLoop, NativeLoop
    import workloads as W

    Hq, Hkv, D, B, N = 32, 8, 128, 16, 16162
    if args.kv_dtype == "fp8":
        return run_serve_fp8(args, torch, np, pkv, DecodeLoop, W, Hq, Hkv, D, B, N)
    rng = np.random.default_rng(11)
    trace = W.request_trace(rng, args.serve_requests)
    max_len = max(p + m for _, p, m in trace)
    order = rng.permutation(N).astype(np.int32)
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1011)
    rows = 1 << 16
    kv_rows = torch.randn((2, rows, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    q_rows = torch.randn((rows, Hq, D), generator=gen, device=dev).to(torch.bfloat16)

    def native(**kw):
        loop = NativeLoop(num_blocks=N, block_size=B, q_heads=Hq, kv_heads=Hkv, head_dim=D,
                          max_running=args.serve_running, free_order=order, **kw)
        loop.set_source(q_rows, kv_rows[0], kv_rows[1], 104729, 7919)
        return loop

    def drive(loop):
        """Run a loop to the end of its trace; the step's account from the
        native step info, the host's busy time per step (the call minus its
        waits for the device) and the device's time per step (HIP events
        around the whole run on the loop's stream)."""
        acc = dict(steps=0, tokens=0, preempted=0, prefill=0, swapped=0, blocks_out=0,
                   blocks_in=0, cached=0, util_sum=0.0, host_us=0.0, wait_us=0.0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        t0 = time.perf_counter()
        while not loop.idle():
            info = loop.step()
            acc["steps"] += 1
            acc["tokens"] += info.n_batch
            acc["preempted"] += info.n_preempted
            acc["prefill"] += info.n_prefill_rows
            acc["swapped"] += info.n_swapped_out
            acc["blocks_out"] += info.n_swap_out_blocks
            acc["blocks_in"] += info.n_swap_in_blocks
            acc["cached"] += info.cached_tokens
            acc["host_us"] += info.host_us
            acc["wait_us"] += info.wait_us
            if info.n_batch:
                acc["util_sum"] += info.tokens_held / max(info.slots_committed, 1)
        e1.record()
        torch.cuda.synchronize()
        acc["wall"] = time.perf_counter() - t0
        acc["device_us"] = e0.elapsed_time(e1) * 1e3
        return acc

    # untimed warm-up: one whole pass of the same trace, so first launches, the
    # loop's buffers and the device allocator's cache (the first step admits
    # over 600 prompts at once) are set up before any timed pass
    warm = native(max_len=max_len)
    for rid, p_, m_ in trace:
        warm.add_request(rid, p_, m_)
    drive(warm)
    warm.close()
    del warm

    block_bytes = 2 * Hkv * D * B * 2          # K and V of one block, bf16
    swap_probe = _swap_probe(torch, pkv, Hkv, D, B, N)
    log(f"bench: swap_blocks probe: {swap_probe}")

    result = {}
    prompts = sum(p_ for _, p_, _ in trace)
    for policy in ("paged", "swap", "reserve"):
        loop = native(max_len=max_len, reserve_max=(policy == "reserve"),
                      host_blocks=N if policy == "swap" else 0)
        for rid, p_, m_ in trace:
            loop.add_request(rid, p_, m_)
        a = drive(loop)
        steps = a["steps"]
        result[policy] = {
            "decode_tokens": a["tokens"], "steps": steps,
            "mean_batch": round(a["tokens"] / steps, 1),
            "preemptions": a["preempted"] + a["swapped"], "dropped": a["preempted"],
            "swapped_out": a["swapped"], "blocks_swapped_out": a["blocks_out"],
            "blocks_swapped_in": a["blocks_in"],
            "swap_bytes": (a["blocks_out"] + a["blocks_in"]) * block_bytes,
            "prefill_tokens_written": a["prefill"],
            "prefill_tokens_recomputed": a["prefill"] - prompts,
            "kv_utilization": round(a["util_sum"] / steps, 4),
            "wall_s": round(a["wall"], 3),
            "decode_tokens_per_s": round(a["tokens"] / a["wall"], 1),
            "host_busy_us_per_step": round((a["host_us"] - a["wait_us"]) / steps, 1),
            "host_wait_us_per_step": round(a["wait_us"] / steps, 1),
            "device_us_per_step": round(a["device_us"] / steps, 1),
        }
        log(f"bench: serve {policy}: {result[policy]}")
        loop.close()
        del loop
    # the same paged pass driven step by step from Python (DecodeLoop), for
    # the host cost of a Python driver against the one native call
    stage = _PinnedIndex(torch, dev)

    def kv_source(pairs):
        idx = stage((pairs[:, 0] * 7919 + pairs[:, 1]) % rows)
        return kv_rows[0].index_select(0, idx), kv_rows[1].index_select(0, idx)

    def q_source(pairs):
        idx = stage((pairs[:, 0] * 104729 + pairs[:, 1]) % rows)
        return q_rows.index_select(0, idx)

    loop = DecodeLoop(num_blocks=N, block_size=B, q_heads=Hq, kv_heads=Hkv, head_dim=D,
                      max_running=args.serve_running, max_len=max_len, free_order=order)
    for rid, p_, m_ in trace:
        loop.add_request(rid, p_, m_)
    py_steps = py_tokens = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while not loop.idle():
        st, _, _, _ = loop.step(kv_source, q_source)
        py_steps += 1
        py_tokens += len(st["batch"])
    torch.cuda.synchronize()
    py_wall = time.perf_counter() - t0
    python_driver = {"steps": py_steps, "wall_s": round(py_wall, 3),
                     "decode_tokens_per_s": round(py_tokens / py_wall, 1),
                     "wall_us_per_step": round(py_wall / py_steps * 1e6, 1)}
    log(f"bench: serve paged, Python driver: {python_driver}")
    del loop
    # prefix caching and chunked prefill: prompts drawn from 8 shared system
    # prompts plus a request-specific part, with a prefill budget per step
    ptrace = W.prefix_trace(np.random.default_rng(12), args.serve_requests, n_prefixes=8,
                            prefix_median=512, suffix_median=96, out_median=128,
                            max_prefix=1024, max_suffix=512, max_out=512, vocab=32000)
    p_max_len = max(p_ + m_ for _, p_, m_, _ in ptrace)
    prefix_result = {}
    for mode in ("cache_off", "cache_on"):
        loop = native(max_len=p_max_len, max_prefill_tokens=args.serve_prefill_budget)
        for rid, p_, m_, toks in ptrace:
            loop.add_request(rid, p_, m_, tokens=toks if mode == "cache_on" else None)
        a = drive(loop)
        prefix_result[mode] = {"steps": a["steps"], "decode_tokens": a["tokens"],
                               "prefill_tokens_computed": a["prefill"],
                               "prompt_tokens_from_cache": a["cached"],
                               "wall_s": round(a["wall"], 3),
                               "decode_tokens_per_s": round(a["tokens"] / a["wall"], 1),
                               "host_busy_us_per_step": round((a["host_us"] - a["wait_us"]) /
                                                              a["steps"], 1),
                               "device_us_per_step": round(a["device_us"] / a["steps"], 1)}
        log(f"bench: serve prefix {mode}: {prefix_result[mode]}")
        loop.close()
        del loop

    rec = {
        "metric": "continuous-batching decode tokens/s, one attention layer (wall clock, "
                  "host scheduling included)",
        "value": result["paged"]["decode_tokens_per_s"],
        "unit": "tokens/s",
        "higher_is_better": True,
        "n_gpus": 1,
        "data": "synthetic",
        "config": {"workload": f"request trace: {len(trace)} requests, prompt log-normal "
                               f"(median 256, sigma 1.0, <= 2048), output log-normal (median "
                               f"256, sigma 0.8, <= 1024), all submitted at start; Llama-3-"
                               f"8B-shaped layer (32/8 heads, D 128, B 16, bf16), {N} blocks, "
                               f"at most {args.serve_running} running",
                   "requests": len(trace), "pool_blocks": N,
                   "max_running": args.serve_running},
        "driver": "one native call per step (pkv_loop_step)",
        "paged": result["paged"],
        "paged_python_driver": python_driver,
        "paged_swap": result["swap"],
        "reserve_max_len": result["reserve"],
        "swap_blocks_probe": swap_probe,
        "prefix_cache": {"workload": f"{len(ptrace)} requests: one of 8 shared prompts "
                                     f"(log-normal median 512 tokens, <= 1024) + a private "
                                     f"part (median 96, <= 512), output median 128; prefill "
                                     f"budget {args.serve_prefill_budget} tokens per step",
                         **prefix_result},
        "paged_vs_reserve_steps": round(result["reserve"]["steps"] / result["paged"]["steps"],
                                        3),
        "paged_vs_reserve_mean_batch": round(result["paged"]["mean_batch"] /
                                             result["reserve"]["mean_batch"], 3),
    }
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


def run_serve_fp8(args, torch, np, pkv, DecodeLoop, W, Hq, Hkv, D, B, N):
    """The continuous-batching loop over fp8 E4M3 pools (the same request trace
    as the bf16 run) at the bf16 pool's block count and at its byte budget
    (twice the blocks), against bf16 at the same byte budget.  Paged policy,
    preemption by dropping and recomputing.  One JSON line."""
    rng = np.random.default_rng(11)
    trace = W.request_trace(rng, args.serve_requests)
    max_len = max(p + m for _, p, m in trace)
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1011)
    rows = 1 << 16
    kv_rows = torch.randn((2, rows, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    q_rows = torch.randn((rows, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
    scales = (torch.full((Hkv,), 0.025, device=dev), torch.full((Hkv,), 0.025, device=dev))

    def run(kv, blocks):
        from paged_kv_cache_346_amd.serve import NativeLoop
        kw = {"dtype": torch.uint8, "kv_scales": scales} if kv == "fp8" else {}
        order = np.random.default_rng(13).permutation(blocks).astype(np.int32)
        loop = NativeLoop(num_blocks=blocks, block_size=B, q_heads=Hq, kv_heads=Hkv, head_dim=D,
                          max_running=args.serve_running, max_len=max_len, free_order=order,
                          **kw)
        loop.set_source(q_rows, kv_rows[0], kv_rows[1], 104729, 7919)
        for rid, p_, m_ in trace:
            loop.add_request(rid, p_, m_)
        steps = tokens = preempted = 0
        host_us = wait_us = 0.0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while not loop.idle():
            info = loop.step()
            steps += 1
            tokens += info.n_batch
            preempted += info.n_preempted
            host_us += info.host_us
            wait_us += info.wait_us
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        loop.close()
        del loop
        return {"kv_dtype": kv, "pool_blocks": blocks,
                "pool_bytes": 2 * blocks * Hkv * D * B * (1 if kv == "fp8" else 2),
                "decode_tokens": tokens, "steps": steps,
                "mean_batch": round(tokens / steps, 1), "preemptions": preempted,
                "wall_s": round(wall, 3), "decode_tokens_per_s": round(tokens / wall, 1),
                "host_busy_us_per_step": round((host_us - wait_us) / steps, 1)}

    run("fp8", N)                               # untimed warm-up passes
    run("bf16", N)
    res = {"bf16": run("bf16", N), "fp8_same_blocks": run("fp8", N),
           "fp8_same_bytes": run("fp8", 2 * N)}
    for k_, v_ in res.items():
        log(f"bench: serve fp8 {k_}: {v_}")
    rec = {
        "metric": "continuous-batching decode tokens/s over fp8 KV, one attention layer "
                  "(wall clock, host scheduling included)",
        "value": res["fp8_same_bytes"]["decode_tokens_per_s"], "unit": "tokens/s",
        "higher_is_better": True, "n_gpus": 1, "data": "synthetic",
        "config": {"workload": f"the bf16 serve trace ({len(trace)} requests); Llama-3-8B-shaped "
                               f"layer (32/8 heads, D 128, B 16); paged, drop + recompute; fp8 "
                               f"E4M3 pools with per-head scales, bf16 rows; one native call "
                               f"per step",
                   "requests": len(trace), "max_running": args.serve_running},
        **res,
    }
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, AMD's published figure


def run_prefill(args, torch, np):
    """Multi-token queries (chunked prefill) over the paged cache: S sequences of
    the Llama-3-8B-shaped layer, each with a cached prefix and a chunk of new
    tokens attending causally over prefix + chunk.  One JSON line (not the
    headline metric); the kernel is timed with HIP events on its launch stream."""
    import paged_kv_cache_346_amd as pkv

    Hq, Hkv, D, B = 32, 8, 128, 16
    S, prefix, chunk = args.prefill_seqs, args.prefill_prefix, args.prefill_chunk
    L = prefix + chunk
    nb = -(-L // B)
    N = S * nb
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(2027)
    fp8 = args.kv_dtype == "fp8"
    pdt = torch.uint8 if fp8 else torch.bfloat16
    ks, vs = pkv.pool_shapes(N, Hkv, D, B, pdt)
    if fp8:
        # finite E4M3 codes of magnitude below 4, random sign; per-head scales
        def codes(shape):
            mag = torch.randint(0, 0x50, shape, generator=gen, device=dev, dtype=torch.uint8)
            return mag | (torch.randint(0, 2, shape, generator=gen, device=dev,
                                        dtype=torch.uint8) << 7)
        k, v = codes(ks), codes(vs)
        scales = {"k_scale": torch.full((Hkv,), 0.025, device=dev),
                  "v_scale": torch.full((Hkv,), 0.025, device=dev)}
    else:
        k = torch.randn(ks, generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn(vs, generator=gen, device=dev).to(torch.bfloat16)
        scales = {}
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(3)).to(torch.int32)
    tables = perm.view(S, nb).to(dev)
    lens = torch.full((S,), L, dtype=torch.int32, device=dev)
    starts = (torch.arange(S + 1, dtype=torch.int32) * chunk).to(dev)
    T = S * chunk
    q = torch.randn((T, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    call = lambda: pkv.paged_attention_prefill(out, q, k, v, tables, lens, starts, chunk,
                                               **scales)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3
    # two contractions (q.K and p.V) of D multiply-adds per (row, head, visible token)
    visible = sum(prefix + i + 1 for i in range(chunk))
    flops = 4.0 * D * Hq * S * visible
    tflops = flops / (us * 1e-6) / 1e12
    kv_bytes = S * L * Hkv * D * 2 * (1 if fp8 else 2)
    kv_desc = "fp8 E4M3 KV with per-head scales, bf16 queries" if fp8 else "bf16"
    rec = {
        "metric": "multi-token query (chunked prefill) attention TFLOP/s",
        "value": round(tflops, 1), "unit": "TFLOP/s", "higher_is_better": True,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{S} sequences x ({prefix} cached + {chunk} new tokens), Llama-3-"
                               f"8B-shaped layer (32/8 heads, D 128, B 16, {kv_desc}), causal "
                               f"over prefix + chunk", "seqs": S, "prefix": prefix, "chunk": chunk,
                   "kv_dtype": "fp8_e4m3" if fp8 else "bf16"},
        "kernel_us": round(us, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "pa_prefill_shared_kernel",
                     "algorithmic_flops_per_launch": flops},
        "kv_bytes_per_launch": kv_bytes,
    }
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="llama8b_gqa", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8"), default=None,
                    help="fp8: the same workload over fp8 E4M3 pools with per-head scales "
                         "(bf16 workloads only; queries and new tokens stay bf16)")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="override the workload's partition size (tokens per workgroup)")
    ap.add_argument("--separate-cache-write", action="store_true",
                    help="write the step's tokens with reshape_and_cache instead of the "
                         "attention launch")
    ap.add_argument("--no-plan", action="store_true",
                    help="launch without the host work plan (one wave per possible partition)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="measure only --config (by default the 70B-shaped batches at both "
                         "block sizes are measured too and reported under 'also')")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--layers", type=int, default=0,
                    help="K/V pools the steps rotate through (0 = enough for 4 GiB)")
    ap.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--serve", action="store_true",
                    help="run the continuous-batching loop over a request trace instead")
    ap.add_argument("--prefill", action="store_true",
                    help="time multi-token queries (chunked prefill) instead")
    ap.add_argument("--prefill-seqs", type=int, default=16)
    ap.add_argument("--prefill-prefix", type=int, default=1536)
    ap.add_argument("--prefill-chunk", type=int, default=512)
    ap.add_argument("--serve-requests", type=int, default=1024)
    ap.add_argument("--serve-running", type=int, default=1024)
    ap.add_argument("--serve-prefill-budget", type=int, default=2048,
                    help="prefill tokens per step in the prefix-cache scenario")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this PagedAttention decode path has no "
              "multi-GPU mode (decode attention shards over sequences and KV heads with no "
              "exchange).  Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.serve:
        return run_serve(args, torch, np)
    if args.prefill:
        return run_prefill(args, torch, np)
    import paged_kv_cache_346_amd as pkv
    import workloads as W

    name = args.config
    rec = measure(args, torch, np, pkv, W, name, args.kv_dtype, primary=True)
    batch = rec.pop("_batch")
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a sample")
        rec["cpu_baseline"] = cpu_baseline(batch, torch, args.cpu_seconds)
    del batch
    if not args.no_extra:
        # the other single-GPU configuration of the >= 70% target (the 70B-shaped
        # long-context batch at both block sizes), measured in the same run, each
        # in a process of its own: a serving process allocates its pool once, and
        # a workload measured after another one's multi-GB pools were allocated
        # and freed in the same process runs 3-4% slower
        rec["also"] = {}
        for other in ("long70b_b16", "long70b_b32"):
            if other == name:
                continue
            r = measure_in_child(args, other)
            rec["also"][other] = {
                "workload": r["config"]["workload"], "value": r["value"], "unit": "GB/s",
                "frac_of_hbm_peak": r["frac_of_hbm_peak"], "ms_per_step": r["ms_per_step"],
                "decode_tokens_per_s": r["decode_tokens_per_s"],
                "main_kernel_GBps": r["roofline"]["achieved"],
                "main_kernel_frac": r["roofline"]["frac"],
                "main_kernel_us": r["roofline"]["launch_us"], "kernel_us": r["kernel_us"],
                "kv_bytes_per_step": r["config"]["kv_bytes_per_step"],
                "partition_size": r["config"]["partition_size"],
                "merge": r["config"]["merge"]}
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


def measure_in_child(args, name):
    """One more workload, measured by this script in a child process with the
    same steps, warm-up and KV dtype; returns its JSON record."""
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "rec.json")
        cmd = [sys.executable, os.path.abspath(__file__), "--config", name, "--no-extra",
               "--no-cpu-baseline", "--steps", str(args.steps), "--warmup", str(args.warmup),
               "--json-out", out]
        if args.kv_dtype:
            cmd += ["--kv-dtype", args.kv_dtype]
        if args.no_plan:
            cmd += ["--no-plan"]
        log(f"bench: measuring {name} in a child process")
        r = subprocess.run(cmd, stdout=subprocess.DEVNULL)
        if r.returncode != 0:
            raise RuntimeError(f"bench.py for {name} exited with {r.returncode}")
        with open(out) as f:
            return json.load(f)


def measure(args, torch, np, pkv, W, name, kv_dtype, primary):
    """Warm-up, the K timed steps and the per-kernel breakdown of one workload;
    returns the JSON record, which also carries the batch (for the CPU
    baseline) under "_batch"."""
    log(f"bench: building workload {name}")
    batch = Batch(pkv, torch, W, name, args.partition_size if primary else None, args.layers,
                  not args.no_plan, not args.separate_cache_write, kv_dtype)
    c = batch.cfg
    log(f"bench: N={batch.w.num_blocks} blocks, KV {batch.kv_bytes / 1e6:.1f} MB, "
        f"{batch.n_pairs} CoW pairs, max L {batch.mcl}")

    if primary and args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"bench: copy probe of {args.copy_probe_mib} MiB done")

    for i in range(args.warmup):
        batch.step(pkv, i)
    torch.cuda.synchronize()

    # contract timing: K steps back to back.  Two events bracket the main-kernel
    # launch of every EVENT_EVERY-th step, on the stream it runs on (torch's
    # current stream, which the binding passes to the library); a pair of event
    # records costs the stream a few microseconds of dispatch gap, so they are
    # not put around every step
    sampled = list(range(0, args.steps, EVENT_EVERY))
    mev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        batch.step(pkv, args.warmup + i, main_ev=mev.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("bench: timed steps done")
    k1_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in mev.values()]))

    def avg_ms(evlist, i):
        return float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evlist]))

    # per-kernel breakdown (untimed pass): regions with no launch are reported as null
    n_bd = min(args.steps, 20)
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_bd)]
    for i in range(n_bd):
        batch.step(pkv, i, ev=bev[i])
    torch.cuda.synchronize()
    names = ("copy_blocks", "reshape_and_cache", "attention_main", "attention_reduce")
    kernel_us = {n: (round(avg_ms(bev, i) * 1e3, 2) if used else None)
                 for i, (n, used) in enumerate(zip(names, batch.launches()))}

    ms_per_step = wall * 1e3 / args.steps
    value = batch.kv_bytes * args.steps / wall / 1e9
    k1_gbs = batch.kv_bytes / (k1_ms * 1e-3) / 1e9
    traffic_key = name + (":fp8" if batch.fp8 else "")
    traffic = load_traffic(traffic_key, 1)
    roofline = {
        "bound": "hbm",
        "achieved": round(k1_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": "pa_mfma_kernel" if (c.dtype == "bf16" and c.G >= 4) else "pa_valu_kernel",
        "traffic_key": traffic_key,
        "launch_us": round(k1_ms * 1e3, 2),
        "launches_timed": len(mev),
        "algorithmic_bytes_per_launch": batch.kv_bytes,
    }
    launches = batch.launches()
    cfg_obj = {
        "workload": f"{name}: {DESCRIPTIONS[name]}" + (
            "; KV pools in fp8 E4M3 with per-KV-head scales (finite codes below 4 in "
            "magnitude), bf16 queries and new tokens" if batch.fp8 else ""),
        "seqs": c.S, "q_heads": c.Hq, "kv_heads": c.Hkv, "head_dim": c.D, "block_size": c.B,
        "kv_dtype": "fp8_e4m3" if batch.fp8 else c.dtype,
        "context_tokens": int(batch.lens_host.sum()),
        "max_context": batch.mcl, "pool_blocks": batch.w.num_blocks,
        "partition_size": batch.P or 512, "new_tokens": 0 if batch.slots is None
        else int(batch.slots.shape[0]), "cow_copies": batch.n_pairs,
        "kv_bytes_per_step": batch.kv_bytes,
        "shared_block_entries": batch.shared_entries,
        "host_plan": batch.plan is not None,
        "cache_write": ("none" if batch.slots is None else
                        "in the attention launch" if batch.append else "reshape_and_cache"),
        "merge": ("reduce launch" if launches[3] else
                  "in the main launch" if batch.mcl > (batch.P or 512) else "none"),
        "work_items": None if batch.plan is None else batch.plan.n_items,
        "pool_bytes_per_layer": batch.pool_bytes,
    }
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": cfg_obj,
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(c.S / (ms_per_step * 1e-3), 1),
        "kernel_us": kernel_us,
        "layers": batch.layers,
        "host_bookkeeping_us": round(batch.host_bookkeeping_us, 1),
        "host_plan_us": None if batch.plan is None else round(batch.host_plan_us, 1),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    rec["_batch"] = batch
    return rec


if __name__ == "__main__":
    sys.exit(main())
