"""Shared set-up for the GPU parity tests: run a workload's request script
through the product's block manager and through the oracle's, require the two
to agree exactly (tables, lengths, slots, copy pairs), poison every slot that
holds no token with NaN, run the device path on the product's bookkeeping, and
run the oracle on its own."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as W
from oracle.attention import paged_attention_decode as ref_decode, valid_slot_mask
from oracle.block_manager import BlockManager as RefBM
from oracle.cache_ops import copy_blocks as ref_copy, reshape_and_cache as ref_cache

NAN_BF16 = np.uint16(0x7FC1)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def poison(k_pool, v_pool, tables, lens, B):
    mask = valid_slot_mask(tables, lens, k_pool.shape[0], B)
    bi, oi = np.nonzero(~mask)
    nan = NAN_BF16 if k_pool.dtype == np.uint16 else np.float32("nan")
    k_pool[bi, :, :, oi, :] = nan
    v_pool[bi, :, :, oi] = nan


def _run_script(bm, ops):
    for op in ops:
        if op[0] == "add":
            bm.add_seq(op[1], op[2])
        elif op[0] == "fork":
            bm.fork(op[1], op[2])
        elif op[0] == "extend":
            for _ in range(op[2]):
                bm.append_slot(op[1])


class Bookkeeping:
    """A workload's request script and step appends, taken through the product's
    block manager and through the oracle's.  The product's tables, lengths,
    slots and copy pairs drive the device; the oracle's drive the oracle; the
    two are asserted equal."""

    def __init__(self, pkv, w: W.Workload):
        c = w.cfg
        ids = list(range(c.S))
        self.max_blocks = max(1, max(-(-int(L) // c.B) for L in w.lengths))
        bm = pkv.BlockManager(w.num_blocks, c.B, w.free_order)
        _run_script(bm, w.ops)
        self.pre_tables, self.pre_lens = bm.fill_batch(ids, self.max_blocks)
        if w.step_ids:
            self.slots, self.pairs = bm.append_slots(w.step_ids)
        else:
            self.slots = np.zeros(0, np.int64)
            self.pairs = np.zeros((0, 2), np.int32)
        self.tables, self.lens = bm.fill_batch(ids, self.max_blocks)
        assert self.lens.tolist() == w.lengths.tolist()
        self.bm = bm

        ref = RefBM(w.num_blocks, c.B, w.free_order)
        _run_script(ref, w.ops)
        pre_t, pre_l = ref.fill_batch(ids, self.max_blocks)
        self.ref_pre_tables = np.asarray(pre_t, np.int32)
        self.ref_pre_lens = np.asarray(pre_l, np.int32)
        appends = [ref.append_slot(s) for s in w.step_ids]
        self.ref_slots = np.asarray([a[0] for a in appends], np.int64)
        self.ref_pairs = np.asarray([[a[1], a[2]] for a in appends if a[1] >= 0],
                                    np.int32).reshape(-1, 2)
        t, l = ref.fill_batch(ids, self.max_blocks)
        self.ref_tables, self.ref_lens = np.asarray(t, np.int32), np.asarray(l, np.int32)
        assert np.array_equal(self.pre_tables, self.ref_pre_tables)
        assert np.array_equal(self.pre_lens, self.ref_pre_lens)
        assert np.array_equal(self.slots, self.ref_slots)
        assert np.array_equal(np.asarray(self.pairs).reshape(-1, 2), self.ref_pairs)
        assert np.array_equal(self.tables, self.ref_tables)
        assert np.array_equal(self.lens, self.ref_lens)


class Case:
    """A workload taken through both block managers (host side only)."""

    def __init__(self, pkv, w: W.Workload, poison_unused: bool = True):
        self.w = w
        c = w.cfg
        bk = Bookkeeping(pkv, w)
        self.bk = bk
        self.max_blocks = bk.max_blocks
        self.slots, self.pairs = bk.slots, bk.pairs
        self.tables, self.lens = bk.tables, bk.lens
        self.k_pool, self.v_pool = w.k_pool, w.v_pool
        if poison_unused:
            self.k_pool, self.v_pool = w.k_pool.copy(), w.v_pool.copy()
            poison(self.k_pool, self.v_pool, bk.ref_pre_tables, bk.ref_pre_lens, c.B)
        self.bm = bk.bm

    # -- device path -----------------------------------------------------------
    def run_device(self, pkv, partition_size=None, shared_kv=None, plan=False, append=False):
        """shared_kv None: set PKV_ATTN_SHARED_KV when the batch shares blocks
        (the benchmark's choice); plan: run from a host work plan; append: let
        the attention launch write the step's tokens (one per sequence, at its
        last position) instead of a separate reshape_and_cache."""
        c = self.w.cfg
        P = c.partition_size if partition_size is None else partition_size
        kp, vp = to_dev(self.k_pool), to_dev(self.v_pool)
        if len(self.pairs):
            pkv.copy_blocks(kp, vp, torch.from_numpy(self.pairs).cuda())
        new_k = new_v = None
        if len(self.slots):
            if append:
                assert list(self.w.step_ids) == list(range(c.S))
                new_k, new_v = to_dev(self.w.k_new), to_dev(self.w.v_new)
            else:
                pkv.reshape_and_cache(to_dev(self.w.k_new), to_dev(self.w.v_new), kp, vp,
                                      torch.from_numpy(self.slots).cuda())
        q = to_dev(self.w.q)
        out = torch.full((c.S, c.Hq, c.D), float("nan"), dtype=torch.float32, device="cuda")
        mcl = int(self.lens.max())
        ws = pkv.attention_workspace(c.S, c.Hq, c.D, mcl, P)
        if shared_kv is None:
            shared_kv = self.bm.count_shared(range(c.S)) > 0
        pl = None
        if plan:
            pl = pkv.make_plan(self.lens, c.Hkv, c.B, self.max_blocks, mcl, P)
        pkv.paged_attention_decode(out, q, kp, vp, torch.from_numpy(self.tables).cuda(),
                                   torch.from_numpy(self.lens).cuda(), mcl, partition_size=P,
                                   workspace=ws, shared_kv=shared_kv, plan=pl,
                                   new_key=new_k, new_value=new_v)
        torch.cuda.synchronize()
        return out.cpu().numpy(), kp, vp

    # -- oracle ----------------------------------------------------------------
    def oracle_pools(self):
        """The oracle's step on the pools, from the oracle's own slots and pairs."""
        kp, vp = self.k_pool, self.v_pool
        bk = self.bk
        if len(bk.ref_pairs):
            kp, vp = ref_copy(kp, vp, bk.ref_pairs)
        if len(bk.ref_slots):
            kp, vp = ref_cache(kp, vp, self.w.k_new, self.w.v_new, bk.ref_slots)
        return kp, vp

    def oracle_out(self, kp, vp, rows=None):
        return ref_decode(self.w.q, kp, vp, self.bk.ref_tables, self.bk.ref_lens, rows=rows)


def check_attention(got: np.ndarray, ref: np.ndarray, dtype: str, rows=None) -> float:
    """Max abs error (bf16) or max per-row relative error (fp32) over the
    compared rows; asserts the stated bound."""
    if rows is None:
        S, H, _ = ref.shape
        rows = [(s, h) for s in range(S) for h in range(H)]
    worst = 0.0
    for s, h in rows:
        g, r = got[s, h].astype(np.float64), ref[s, h]
        assert np.isfinite(g).all(), (s, h)
        err = np.abs(g - r).max()
        if dtype == "bf16":
            worst = max(worst, err)
            assert err <= 2e-3, (s, h, err)
        else:
            rel = err / np.abs(r).max()
            worst = max(worst, rel)
            assert rel <= 1e-5, (s, h, rel)
    return worst
