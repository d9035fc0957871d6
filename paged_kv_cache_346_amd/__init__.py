"""PagedAttention decode for AMD MI355X (gfx950): Python binding of libpkv.so.

Argument marshalling only.  Every step of the path runs inside the library:
the HIP kernels (reshape_and_cache, copy_blocks, paged_attention_decode) and the
host block manager (allocate, free, refcount, fork, copy-on-write).  PyTorch
supplies device memory and the current stream.  The names match the C entry
points declared in include/pkv.h (short aliases without the pkv_ prefix are
provided too).  There is no fallback: if libpkv.so is missing, importing this
package raises ImportError.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch  # imported before the library so both share torch's HIP runtime

__all__ = [
    "PkvError", "BlockManager", "Scheduler", "pkv_reshape_and_cache", "pkv_copy_blocks",
    "pkv_swap_blocks", "swap_blocks", "pkv_paged_attention_prefill", "paged_attention_prefill",
    "pkv_attention_workspace_bytes", "pkv_paged_attention_decode", "pkv_paged_attention_main",
    "pkv_paged_attention_reduce", "pool_shapes", "paged_attention_main", "paged_attention_reduce",
    "pkv_attention_plan", "pkv_attention_plan_words", "attention_plan", "attention_plan_words",
    "Plan", "make_plan", "StepPack", "LoopConfig", "LoopSource", "LoopStepInfo",
    "reshape_and_cache", "copy_blocks", "attention_workspace_bytes", "attention_workspace",
    "paged_attention_decode", "pkv_paged_attention_decode_noalloc",
    "paged_attention_decode_noalloc", "PKV_ENOSCRATCH", "PKV_SCRATCH_BYTES",
    "LIB_PATH", "lib",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_ENOBLOCKS, PKV_ENOSEQ, PKV_EEXIST, PKV_EUNSUPPORTED, PKV_EHIP = (
    0, -1, -2, -3, -4, -5, -6)
PKV_ENOSCRATCH = -7
PKV_SCRATCH_BYTES = 64 << 20
PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
PKV_ATTN_SHARED_KV = 1
PKV_SCHED_RESERVE_MAX, PKV_SCHED_SWAP = 1, 2

_i32, _i64, _f32, _vp, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                              ctypes.c_size_t)
_u32 = ctypes.c_uint32
_pi32, _pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)

class _SchedStep(ctypes.Structure):
    """pkv_sched_step (include/pkv.h)."""
    _fields_ = [("capacity", ctypes.c_int32),
                ("batch_ids", ctypes.POINTER(ctypes.c_int64)),
                ("slots", ctypes.POINTER(ctypes.c_int64)),
                ("n_batch", ctypes.c_int32),
                ("cow_pairs", ctypes.POINTER(ctypes.c_int32)),
                ("n_cow", ctypes.c_int32),
                ("admitted_ids", ctypes.POINTER(ctypes.c_int64)),
                ("admitted_ctx", ctypes.POINTER(ctypes.c_int32)),
                ("admitted_cached", ctypes.POINTER(ctypes.c_int32)),
                ("n_admitted", ctypes.c_int32),
                ("prefill_ids", ctypes.POINTER(ctypes.c_int64)),
                ("prefill_start", ctypes.POINTER(ctypes.c_int32)),
                ("prefill_len", ctypes.POINTER(ctypes.c_int32)),
                ("n_prefill", ctypes.c_int32),
                ("preempted_ids", ctypes.POINTER(ctypes.c_int64)),
                ("n_preempted", ctypes.c_int32),
                ("finished_ids", ctypes.POINTER(ctypes.c_int64)),
                ("n_finished", ctypes.c_int32),
                ("pair_capacity", ctypes.c_int32),
                ("swap_in_pairs", ctypes.POINTER(ctypes.c_int32)),
                ("n_swap_in", ctypes.c_int32),
                ("swap_out_pairs", ctypes.POINTER(ctypes.c_int32)),
                ("n_swap_out", ctypes.c_int32),
                ("swapped_in_ids", ctypes.POINTER(ctypes.c_int64)),
                ("n_swapped_in", ctypes.c_int32),
                ("swapped_out_ids", ctypes.POINTER(ctypes.c_int64)),
                ("n_swapped_out", ctypes.c_int32)]


class StepPack(ctypes.Structure):
    """pkv_step_pack (include/pkv.h): where pkv_pack_step put each array, in
    int32 words from the buffer's start."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "total_words", "n_prefill_rows", "slots_off", "pf_tables_off", "pf_width",
        "pf_lens_off", "pf_start_off", "pf_max_rows", "tables_off", "width", "lens_off",
        "max_context", "plan_off", "n_items", "n_merge", "pairs_off", "swap_in_off",
        "swap_out_off", "cow_off")]


class LoopConfig(ctypes.Structure):
    """pkv_loop_config (include/pkv.h)."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "num_blocks", "block_size", "q_heads", "kv_heads", "head_dim", "max_running", "max_len",
        "partition_size", "host_blocks", "dtype")]


class LoopSource(ctypes.Structure):
    """pkv_loop_source (include/pkv.h): the step's rows from device banks."""
    _fields_ = [("q_bank", ctypes.c_void_p), ("k_bank", ctypes.c_void_p),
                ("v_bank", ctypes.c_void_p), ("bank_rows", ctypes.c_int64),
                ("q_mul", ctypes.c_int64), ("kv_mul", ctypes.c_int64)]


class LoopStepInfo(ctypes.Structure):
    """pkv_loop_step_info (include/pkv.h)."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "n_batch", "n_prefill", "n_prefill_rows", "n_admitted", "n_preempted", "n_finished",
        "n_swapped_out", "n_swapped_in", "n_swap_out_blocks", "n_swap_in_blocks", "n_cow",
        "max_context")] + [
        ("cached_tokens", ctypes.c_int64), ("tokens_held", ctypes.c_int64),
        ("slots_committed", ctypes.c_int64), ("n_waiting", ctypes.c_int32),
        ("n_running", ctypes.c_int32), ("n_swapped", ctypes.c_int32),
        ("lens_host", ctypes.POINTER(ctypes.c_int32)), ("decode_out", ctypes.c_void_p),
        ("prefill_out", ctypes.c_void_p), ("host_us", ctypes.c_double),
        ("wait_us", ctypes.c_double)]


# name -> (restype, argtypes); mirrors include/pkv.h
SIGNATURES = {
    "pkv_status_string": (ctypes.c_char_p, [_i32]),
    "pkv_bm_create": (_i32, [_i32, _i32, _pi32, ctypes.POINTER(_vp)]),
    "pkv_bm_destroy": (None, [_vp]),
    "pkv_bm_add_seq": (_i32, [_vp, _i64, _i32]),
    "pkv_bm_append_slot": (_i32, [_vp, _i64, _pi64, _pi32, _pi32]),
    "pkv_bm_append_slots": (_i32, [_vp, _pi64, _i32, _pi64, _pi32, _pi32, _pi32]),
    "pkv_bm_fork": (_i32, [_vp, _i64, _i64]),
    "pkv_bm_free_seq": (_i32, [_vp, _i64]),
    "pkv_bm_truncate": (_i32, [_vp, _i64, _i32]),
    "pkv_bm_num_free": (_i32, [_vp, _pi32]),
    "pkv_bm_geometry": (_i32, [_vp, _pi32, _pi32]),
    "pkv_sched_create": (_i32, [_vp, _i32, _i32, _i32, ctypes.POINTER(_vp)]),
    "pkv_sched_destroy": (None, [_vp]),
    "pkv_sched_add_request": (_i32, [_vp, _i64, _i32, _i32, _pi32]),
    "pkv_sched_begin_step": (_i32, [_vp, ctypes.POINTER(_SchedStep)]),
    "pkv_sched_end_step": (_i32, [_vp]),
    "pkv_sched_stats": (_i32, [_vp, _pi64, _pi64, _pi32, _pi32, _pi32]),
    "pkv_pack_step": (_i32, [_vp, ctypes.POINTER(_SchedStep), _i32, _i32, _i32, _pi32, _sz,
                             ctypes.POINTER(StepPack)]),
    "pkv_bm_refcount": (_i32, [_vp, _i32, _pi32]),
    "pkv_bm_seq_info": (_i32, [_vp, _i64, _pi32, _pi32]),
    "pkv_bm_block_table": (_i32, [_vp, _i64, _pi32, _i32]),
    "pkv_bm_fill_batch": (_i32, [_vp, _pi64, _i32, _i32, _pi32, _pi32]),
    "pkv_bm_snapshot": (_i32, [_vp, _pi32, _pi32, _pi32]),
    "pkv_bm_add_seq_prefix": (_i32, [_vp, _i64, _pi32, _i32, _i32, _pi32]),
    "pkv_bm_cached_blocks": (_i32, [_vp, _pi32]),
    "pkv_bm_register_prefix": (_i32, [_vp, _i64, _pi32, _i32, _i32]),
    "pkv_bm_unregister_prefix": (_i32, [_vp, _i64, _i32]),
    "pkv_bm_set_host_pool": (_i32, [_vp, _i32]),
    "pkv_bm_num_free_host": (_i32, [_vp, _pi32]),
    "pkv_bm_is_swapped": (_i32, [_vp, _i64, _pi32]),
    "pkv_bm_swap_out": (_i32, [_vp, _i64, _pi32, _i32, _pi32]),
    "pkv_bm_swap_in": (_i32, [_vp, _i64, _pi32, _i32, _pi32]),
    "pkv_bm_host_snapshot": (_i32, [_vp, _pi32, _pi32]),
    "pkv_bm_count_shared": (_i32, [_vp, _pi64, _i32, _pi64]),
    "pkv_bm_slots": (_i32, [_vp, _i64, _i32, _i32, _pi64]),
    "pkv_loop_create": (_i32, [ctypes.POINTER(LoopConfig), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, ctypes.POINTER(_vp)]),
    "pkv_loop_destroy": (None, [_vp]),
    "pkv_loop_copy_outputs": (_i32, [_vp, _vp, _vp]),
    "pkv_loop_step": (_i32, [_vp, ctypes.POINTER(LoopSource), ctypes.POINTER(LoopStepInfo)]),
    "pkv_reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _vp, _vp, _vp]),
    "pkv_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pkv_paged_attention_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                           _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp,
                                           _vp, _vp]),
    "pkv_swap_blocks": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                               _i32, _vp]),
    "pkv_attention_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_attention_plan_words": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_attention_plan": (_i32, [_pi32, _i32, _i32, _i32, _i32, _i32, _i32, _pi32, _sz, _pi32,
                                  _pi32]),
    "pkv_paged_attention_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                          _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp,
                                          _i32, _i32, _vp, _sz, _i32, _u32, _vp, _vp, _vp]),
    "pkv_paged_attention_main": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _i32,
                                        _i32, _vp, _sz, _i32, _u32, _vp, _vp, _vp]),
    "pkv_paged_attention_reduce": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                          _i32, _vp, _i32, _i32, _vp, _sz, _vp]),
    "pkv_paged_attention_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                                  _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                                  _i32, _vp, _i32, _i32, _i32, _u32, _vp, _vp,
                                                  _vp]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python paged_kv_cache_346_amd/build.py`")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


class PkvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = int(code)
        super().__init__(f"{where}: {lib.pkv_status_string(self.code).decode()}")


def _check(code: int, where: str) -> None:
    if code != PKV_OK:
        raise PkvError(code, where)


def _np_ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ---------------------------------------------------------------------------
# host block manager
# ---------------------------------------------------------------------------
class BlockManager:
    """Owner of a pkv_bm handle: the pool's refcounts, free queue and tables."""

    def __init__(self, num_blocks: int, block_size: int, init_free_order=None):
        h = _vp()
        order = None
        if init_free_order is not None:
            order = np.ascontiguousarray(init_free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("init_free_order must hold num_blocks entries")
        _check(lib.pkv_bm_create(num_blocks, block_size,
                                 None if order is None else _np_ptr(order, ctypes.c_int32),
                                 ctypes.byref(h)), "pkv_bm_create")
        self._h = h
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_seq(self, seq_id: int, num_tokens: int) -> None:
        _check(lib.pkv_bm_add_seq(self._h, seq_id, num_tokens), "pkv_bm_add_seq")

    def append_slot(self, seq_id: int):
        slot, src, dst = _i64(), _i32(), _i32()
        _check(lib.pkv_bm_append_slot(self._h, seq_id, ctypes.byref(slot), ctypes.byref(src),
                                      ctypes.byref(dst)), "pkv_bm_append_slot")
        return slot.value, src.value, dst.value

    def append_slots(self, seq_ids):
        """One decode step: (slots int64 [n], cow pairs int32 [k, 2])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        slots = np.empty(n, np.int64)
        pairs = np.empty((max(n, 1), 2), np.int32)
        n_cow, n_done = _i32(), _i32()
        _check(lib.pkv_bm_append_slots(self._h, _np_ptr(ids, ctypes.c_int64), n,
                                       _np_ptr(slots, ctypes.c_int64),
                                       _np_ptr(pairs, ctypes.c_int32), ctypes.byref(n_cow),
                                       ctypes.byref(n_done)), "pkv_bm_append_slots")
        return slots, pairs[:n_cow.value].copy()

    def fork(self, parent_id: int, child_id: int) -> None:
        _check(lib.pkv_bm_fork(self._h, parent_id, child_id), "pkv_bm_fork")

    def free_seq(self, seq_id: int) -> None:
        _check(lib.pkv_bm_free_seq(self._h, seq_id), "pkv_bm_free_seq")

    def truncate(self, seq_id: int, new_len: int) -> None:
        """pkv_bm_truncate: give back the sequence's tokens past new_len."""
        _check(lib.pkv_bm_truncate(self._h, seq_id, new_len), "pkv_bm_truncate")

    def geometry(self):
        """(num_blocks, block_size)."""
        n, b = _i32(), _i32()
        _check(lib.pkv_bm_geometry(self._h, ctypes.byref(n), ctypes.byref(b)), "pkv_bm_geometry")
        return n.value, b.value

    def num_free(self) -> int:
        out = _i32()
        _check(lib.pkv_bm_num_free(self._h, ctypes.byref(out)), "pkv_bm_num_free")
        return out.value

    def refcount(self, block: int) -> int:
        out = _i32()
        _check(lib.pkv_bm_refcount(self._h, block, ctypes.byref(out)), "pkv_bm_refcount")
        return out.value

    def seq_info(self, seq_id: int):
        ln, nb = _i32(), _i32()
        _check(lib.pkv_bm_seq_info(self._h, seq_id, ctypes.byref(ln), ctypes.byref(nb)),
               "pkv_bm_seq_info")
        return ln.value, nb.value

    def block_table(self, seq_id: int):
        _, nb = self.seq_info(seq_id)
        out = np.empty(max(nb, 1), np.int32)
        _check(lib.pkv_bm_block_table(self._h, seq_id, _np_ptr(out, ctypes.c_int32), nb),
               "pkv_bm_block_table")
        return out[:nb].tolist()

    def fill_batch(self, seq_ids, max_blocks: int):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        tables = np.empty((n, max_blocks), np.int32)
        lens = np.empty(n, np.int32)
        _check(lib.pkv_bm_fill_batch(self._h, _np_ptr(ids, ctypes.c_int64), n, max_blocks,
                                     _np_ptr(tables, ctypes.c_int32),
                                     _np_ptr(lens, ctypes.c_int32)), "pkv_bm_fill_batch")
        return tables, lens

    def slots(self, seq_id: int, start: int, count: int) -> np.ndarray:
        """int64 slots of tokens [start, start+count) of a sequence."""
        out = np.empty(max(count, 1), np.int64)
        _check(lib.pkv_bm_slots(self._h, seq_id, start, count, _np_ptr(out, ctypes.c_int64)),
               "pkv_bm_slots")
        return out[:count]

    def count_shared(self, seq_ids) -> int:
        """Table entries of these sequences whose block has refcount > 1."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        out = _i64()
        _check(lib.pkv_bm_count_shared(self._h, _np_ptr(ids, ctypes.c_int64), ids.shape[0],
                                       ctypes.byref(out)), "pkv_bm_count_shared")
        return out.value

    def snapshot(self):
        ref = np.empty(self.num_blocks, np.int32)
        fq = np.empty(self.num_blocks, np.int32)
        nf = _i32()
        _check(lib.pkv_bm_snapshot(self._h, _np_ptr(ref, ctypes.c_int32),
                                   _np_ptr(fq, ctypes.c_int32), ctypes.byref(nf)),
               "pkv_bm_snapshot")
        return ref.tolist(), fq[:nf.value].tolist()

    # -- prefix cache ----------------------------------------------------------
    def add_seq_prefix(self, seq_id: int, tokens, num_tokens: int) -> int:
        """Admit a sequence whose first len(tokens) ids are known, reusing cached
        full blocks of its prefix; returns the tokens already cached."""
        ids = np.ascontiguousarray(tokens, dtype=np.int32)
        out = _i32()
        _check(lib.pkv_bm_add_seq_prefix(self._h, seq_id, _np_ptr(ids, ctypes.c_int32),
                                         ids.shape[0], num_tokens, ctypes.byref(out)),
               "pkv_bm_add_seq_prefix")
        return out.value

    def register_prefix(self, seq_id: int, tokens, upto: int) -> None:
        """Register the sequence's full blocks that the ids cover, up to token upto."""
        ids = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(lib.pkv_bm_register_prefix(self._h, seq_id, _np_ptr(ids, ctypes.c_int32),
                                          ids.shape[0], upto), "pkv_bm_register_prefix")

    def unregister_prefix(self, seq_id: int, start: int) -> None:
        _check(lib.pkv_bm_unregister_prefix(self._h, seq_id, start), "pkv_bm_unregister_prefix")

    def cached_blocks(self) -> int:
        out = _i32()
        _check(lib.pkv_bm_cached_blocks(self._h, ctypes.byref(out)), "pkv_bm_cached_blocks")
        return out.value

    # -- swapping (host pool) ------------------------------------------------
    def set_host_pool(self, num_host_blocks: int) -> None:
        _check(lib.pkv_bm_set_host_pool(self._h, num_host_blocks), "pkv_bm_set_host_pool")
        self.num_host_blocks = int(num_host_blocks)

    def num_free_host(self) -> int:
        out = _i32()
        _check(lib.pkv_bm_num_free_host(self._h, ctypes.byref(out)), "pkv_bm_num_free_host")
        return out.value

    def is_swapped(self, seq_id: int) -> bool:
        out = _i32()
        _check(lib.pkv_bm_is_swapped(self._h, seq_id, ctypes.byref(out)), "pkv_bm_is_swapped")
        return bool(out.value)

    def _swap(self, fn, name, seq_id):
        _, nb = self.seq_info(seq_id)
        pairs = np.empty((max(nb, 1), 2), np.int32)
        n = _i32()
        _check(fn(self._h, seq_id, _np_ptr(pairs, ctypes.c_int32), nb, ctypes.byref(n)), name)
        return pairs[:n.value].copy()

    def swap_out(self, seq_id: int) -> np.ndarray:
        """(device block, host block) pairs int32 [n, 2], table order."""
        return self._swap(lib.pkv_bm_swap_out, "pkv_bm_swap_out", seq_id)

    def swap_in(self, seq_id: int) -> np.ndarray:
        """(host block, device block) pairs int32 [n, 2], table order."""
        return self._swap(lib.pkv_bm_swap_in, "pkv_bm_swap_in", seq_id)

    def host_free_queue(self):
        cap = getattr(self, "num_host_blocks", 0)
        fq = np.empty(max(cap, 1), np.int32)
        nf = _i32()
        _check(lib.pkv_bm_host_snapshot(self._h, _np_ptr(fq, ctypes.c_int32), ctypes.byref(nf)),
               "pkv_bm_host_snapshot")
        return fq[:nf.value].tolist()


class Scheduler:
    """Owner of a pkv_sched handle: continuous batching over a BlockManager
    (which must outlive it).  begin_step() returns the step as a dict with the
    same keys as the reference scheduler: batch, slots, cow, admitted
    [(id, ctx)], preempted, finished, swap_in [(host, device)], swap_out
    [(device, host)], swapped_in, swapped_out."""

    def __init__(self, bm: BlockManager, max_running: int, reserve_max: bool = False,
                 swap: bool = False, max_prefill_tokens=None):
        h = _vp()
        policy = (PKV_SCHED_RESERVE_MAX if reserve_max else 0) | (PKV_SCHED_SWAP if swap else 0)
        _check(lib.pkv_sched_create(bm._h, max_running, policy, int(max_prefill_tokens or 0),
                                    ctypes.byref(h)), "pkv_sched_create")
        self._h, self.bm, self.max_running = h, bm, int(max_running)
        n = self.max_running
        npairs = bm.num_blocks
        self._swin = np.zeros(2 * npairs, np.int32)
        self._swout = np.zeros(2 * npairs, np.int32)
        self._swin_ids = np.zeros(n, np.int64)
        self._swout_ids = np.zeros(n, np.int64)
        self._ids = np.zeros(n, np.int64)
        self._slots = np.zeros(n, np.int64)
        self._cow = np.zeros(2 * n, np.int32)
        self._adm = np.zeros(n, np.int64)
        self._adm_ctx = np.zeros(n, np.int32)
        self._adm_cached = np.zeros(n, np.int32)
        self._pf_ids = np.zeros(n, np.int64)
        self._pf_start = np.zeros(n, np.int32)
        self._pf_len = np.zeros(n, np.int32)
        self._pre = np.zeros(n, np.int64)
        self._fin = np.zeros(n, np.int64)
        self._step = _SchedStep(n, _np_ptr(self._ids, ctypes.c_int64),
                                _np_ptr(self._slots, ctypes.c_int64), 0,
                                _np_ptr(self._cow, ctypes.c_int32), 0,
                                _np_ptr(self._adm, ctypes.c_int64),
                                _np_ptr(self._adm_ctx, ctypes.c_int32),
                                _np_ptr(self._adm_cached, ctypes.c_int32), 0,
                                _np_ptr(self._pf_ids, ctypes.c_int64),
                                _np_ptr(self._pf_start, ctypes.c_int32),
                                _np_ptr(self._pf_len, ctypes.c_int32), 0,
                                _np_ptr(self._pre, ctypes.c_int64), 0,
                                _np_ptr(self._fin, ctypes.c_int64), 0, npairs,
                                _np_ptr(self._swin, ctypes.c_int32), 0,
                                _np_ptr(self._swout, ctypes.c_int32), 0,
                                _np_ptr(self._swin_ids, ctypes.c_int64), 0,
                                _np_ptr(self._swout_ids, ctypes.c_int64), 0)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib.pkv_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_request(self, req_id: int, prompt_len: int, max_new_tokens: int,
                    tokens=None) -> None:
        ids = None
        if tokens is not None:
            ids = np.ascontiguousarray(tokens, dtype=np.int32)
            if ids.shape != (prompt_len,):
                raise ValueError("token ids must cover the prompt")
        _check(lib.pkv_sched_add_request(self._h, req_id, prompt_len, max_new_tokens,
                                         None if ids is None else _np_ptr(ids, ctypes.c_int32)),
               "pkv_sched_add_request")

    def begin_step(self):
        st = self._step
        _check(lib.pkv_sched_begin_step(self._h, ctypes.byref(st)), "pkv_sched_begin_step")
        nb, nc = st.n_batch, st.n_cow
        return {
            "batch": self._ids[:nb].tolist(),
            "slots": self._slots[:nb].tolist(),
            "cow": [tuple(x) for x in self._cow[:2 * nc].reshape(-1, 2).tolist()],
            "admitted": list(zip(self._adm[:st.n_admitted].tolist(),
                                 self._adm_ctx[:st.n_admitted].tolist(),
                                 self._adm_cached[:st.n_admitted].tolist())),
            "prefill": list(zip(self._pf_ids[:st.n_prefill].tolist(),
                                self._pf_start[:st.n_prefill].tolist(),
                                self._pf_len[:st.n_prefill].tolist())),
            "preempted": self._pre[:st.n_preempted].tolist(),
            "finished": self._fin[:st.n_finished].tolist(),
            "swap_in": [tuple(x) for x in self._swin[:2 * st.n_swap_in].reshape(-1, 2).tolist()],
            "swap_out": [tuple(x) for x in self._swout[:2 * st.n_swap_out].reshape(-1, 2).tolist()],
            "swapped_in": self._swin_ids[:st.n_swapped_in].tolist(),
            "swapped_out": self._swout_ids[:st.n_swapped_out].tolist(),
        }

    def end_step(self) -> None:
        _check(lib.pkv_sched_end_step(self._h), "pkv_sched_end_step")

    def pack_step(self, max_blocks: int, Hkv: int, partition_size: int, buf: np.ndarray,
                  out: StepPack) -> bool:
        """pkv_pack_step for the step begin_step just returned, into the int32
        array `buf`; False (with out.total_words set) when buf is too small."""
        st = lib.pkv_pack_step(self.bm._h, ctypes.byref(self._step), max_blocks, Hkv,
                               partition_size, _np_ptr(buf, ctypes.c_int32), buf.shape[0],
                               ctypes.byref(out))
        if st == PKV_EINVAL and out.total_words > buf.shape[0]:
            return False
        _check(st, "pkv_pack_step")
        return True

    def stats(self):
        """(tokens held, slots committed, waiting, running, swapped out)."""
        held, committed, nw, nr, ns = _i64(), _i64(), _i32(), _i32(), _i32()
        _check(lib.pkv_sched_stats(self._h, ctypes.byref(held), ctypes.byref(committed),
                                   ctypes.byref(nw), ctypes.byref(nr), ctypes.byref(ns)),
               "pkv_sched_stats")
        return held.value, committed.value, nw.value, nr.value, ns.value


# ---------------------------------------------------------------------------
# device operations
# ---------------------------------------------------------------------------
_FP8_DTYPES = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype in _FP8_DTYPES:
        return PKV_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16, or uint8 / "
                    f"float8_e4m3fn for fp8 E4M3)")


def _row_dtype(pool: torch.Tensor) -> torch.dtype:
    """dtype of the q / K / V rows that go with a pool (bf16 for fp8 pools)."""
    return torch.bfloat16 if pool.dtype in _FP8_DTYPES else pool.dtype


def _scales(k_pool, k_scale, v_scale, Hkv):
    """Device pointers of the per-head fp8 scales (None for other pools)."""
    if k_pool.dtype not in _FP8_DTYPES:
        return None, None
    for t, name in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t is None or t.dtype != torch.float32 or tuple(t.shape) != (Hkv,):
            raise ValueError(f"fp8 pools need {name}: float32 [Hkv] on the device")
    return _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale")


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def pool_shapes(num_blocks: int, Hkv: int, D: int, B: int, dtype: torch.dtype):
    """Tensor shapes of the K and V pools (K [N, Hkv, D/x, B, x], V [N, Hkv, D, B])."""
    x = 16 // (4 if dtype == torch.float32 else 1 if dtype in _FP8_DTYPES else 2)
    return (num_blocks, Hkv, D // x, B, x), (num_blocks, Hkv, D, B)


def _pool_geometry(k_pool: torch.Tensor, v_pool: torch.Tensor):
    if k_pool.dim() != 5 or v_pool.dim() != 4:
        raise ValueError("k_pool must be [N, Hkv, D/x, B, x] and v_pool [N, Hkv, D, B]")
    N, Hkv, Dx, B, x = k_pool.shape
    D = Dx * x
    if tuple(v_pool.shape) != (N, Hkv, D, B) or k_pool.dtype != v_pool.dtype:
        raise ValueError("k_pool and v_pool disagree in shape or dtype")
    if x * k_pool.element_size() != 16:
        raise ValueError("k_pool's last dim must span 16 bytes")
    return N, Hkv, D, B


def pkv_reshape_and_cache(key, value, k_pool, v_pool, slot_mapping, stream=None,
                          k_scale=None, v_scale=None) -> None:
    """Write token i's K/V ([T, Hkv, D]) into slot slot_mapping[i] (int64; <0 skips).
    fp8 pools: key/value are bf16 and are encoded with the per-head scales
    (float32 [Hkv] device tensors)."""
    N, Hkv, D, B = _pool_geometry(k_pool, v_pool)
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D):
        raise ValueError("key/value must be [T, Hkv, D]")
    if key.dtype != _row_dtype(k_pool) or value.dtype != _row_dtype(k_pool):
        raise ValueError("key/value dtype must match the pools (bf16 for fp8 pools)")
    if slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    ks, vs = _scales(k_pool, k_scale, v_scale, Hkv)
    _check(lib.pkv_reshape_and_cache(_dev(key, "key"), _dev(value, "value"),
                                     _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                     _dev(slot_mapping, "slot_mapping"), T, Hkv, D, B, N,
                                     _dtype_code(k_pool), ks, vs, _stream(stream)),
           "pkv_reshape_and_cache")


def pkv_copy_blocks(k_pool, v_pool, pairs, stream=None) -> None:
    """Copy block pairs[k, 0] onto pairs[k, 1] in both pools (int32 [n, 2] on device)."""
    N, Hkv, D, B = _pool_geometry(k_pool, v_pool)
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int32 [n, 2]")
    n = pairs.shape[0]
    if n == 0:
        return
    _check(lib.pkv_copy_blocks(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                               _dev(pairs, "pairs"), n, Hkv, D, B, N, _dtype_code(k_pool),
                               _stream(stream)), "pkv_copy_blocks")


def _pool_ptr(t: torch.Tensor, name: str) -> int:
    """Device tensor, or pinned host tensor (the library maps it for the GPU)."""
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda and not t.is_pinned():
        raise ValueError(f"{name} must be a device tensor or a pinned host tensor")
    return t.data_ptr()


def pkv_swap_blocks(dst_k, dst_v, src_k, src_v, pairs, stream=None) -> None:
    """dst block pairs[k, 1] := src block pairs[k, 0] (K and V), between two pools
    of the same geometry, each on the device or in pinned host memory; pairs is
    int32 [n, 2] on the device."""
    N_dst, Hkv, D, B = _pool_geometry(dst_k, dst_v)
    N_src, *geo = _pool_geometry(src_k, src_v)
    if tuple(geo) != (Hkv, D, B) or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination pools differ in geometry or dtype")
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int32 [n, 2]")
    n = pairs.shape[0]
    if n == 0:
        return
    _check(lib.pkv_swap_blocks(_pool_ptr(dst_k, "dst_k"), _pool_ptr(dst_v, "dst_v"), N_dst,
                               _pool_ptr(src_k, "src_k"), _pool_ptr(src_v, "src_v"), N_src,
                               _dev(pairs, "pairs"), n, Hkv, D, B, _dtype_code(dst_k),
                               _stream(stream)), "pkv_swap_blocks")


def pkv_paged_attention_prefill(out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                                max_query_len: int, scale=None, stream=None, k_scale=None,
                                v_scale=None) -> None:
    """Causal attention of each sequence's last Q_s tokens over the paged cache:
    q and out [T, Hq, D] packed by query_start (int32 [S+1]); Q_s =
    query_start[s+1] - query_start[s].  fp8 pools take bf16 q and the per-head
    k_scale / v_scale (float32 [Hkv] device tensors).

    max_query_len bounds every Q_s and sizes the grid.  query_start may be a
    host array (numpy or a CPU tensor): it is then checked against that bound
    (ValueError when some Q_s exceeds it) and copied to the device.  A device
    query_start is not read on the host; there an undersized bound leaves a
    sequence's earliest rows unwritten."""
    N, Hkv, D, B = _pool_geometry(k_pool, v_pool)
    T, Hq = q.shape[0], q.shape[1]
    S = context_lens.shape[0]
    if tuple(q.shape) != (T, Hq, D) or tuple(out.shape) != (T, Hq, D):
        raise ValueError("q and out must be [T, Hq, D]")
    if out.dtype != torch.float32 or q.dtype != _row_dtype(k_pool):
        raise ValueError("out must be fp32 and q in the pool dtype (bf16 for fp8 pools)")
    if not (isinstance(query_start, torch.Tensor) and query_start.is_cuda):
        qs = query_start.numpy() if isinstance(query_start, torch.Tensor) else query_start
        qs = np.ascontiguousarray(qs, dtype=np.int32)
        if qs.shape != (S + 1,):
            raise ValueError("query_start must be int32 [S + 1]")
        longest = int(np.diff(qs).max()) if S > 0 else 0
        if longest > int(max_query_len):
            raise ValueError(f"max_query_len {int(max_query_len)} is below the longest "
                             f"query run in query_start ({longest} rows)")
        query_start = torch.from_numpy(qs).to(out.device)
    if query_start.dtype != torch.int32 or tuple(query_start.shape) != (S + 1,):
        raise ValueError("query_start must be int32 [S + 1]")
    if context_lens.dtype != torch.int32 or block_tables.dtype != torch.int32 or \
            block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [S, max_blocks], context_lens int32 [S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if S == 0 or T == 0:
        return
    _check(lib.pkv_paged_attention_prefill(
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
        _dev(query_start, "query_start"), S, T, Hq, Hkv, D, B, block_tables.shape[1], N,
        int(max_query_len), float(scale), _dtype_code(k_pool),
        *_scales(k_pool, k_scale, v_scale, Hkv), _stream(stream)),
        "pkv_paged_attention_prefill")


def pkv_attention_workspace_bytes(S: int, Hq: int, D: int, max_context_len: int,
                                  partition_size: int = 0) -> int:
    return int(lib.pkv_attention_workspace_bytes(S, Hq, D, max_context_len, partition_size))


def attention_workspace(S: int, Hq: int, D: int, max_context_len: int, partition_size: int = 0,
                        device="cuda") -> torch.Tensor:
    """A zeroed uint8 device workspace of pkv_attention_workspace_bytes (at least
    16 bytes).  Its first 64 KiB hold the in-launch merge's counters, which
    must be zero before the first call; every call leaves them zero, so one
    workspace serves any number of calls of at most this size."""
    n = pkv_attention_workspace_bytes(S, Hq, D, max_context_len, partition_size)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


class Plan:
    """A device copy of a host work plan (pkv_attention_plan) and its counts."""

    def __init__(self, words: torch.Tensor, n_items: int, n_merge: int):
        if words.dtype != torch.int32 or not words.is_cuda:
            raise ValueError("plan words must be an int32 device tensor")
        self.words, self.n_items, self.n_merge = words, int(n_items), int(n_merge)


def pkv_attention_plan_words(S: int, Hkv: int, B: int, max_blocks: int, max_context_len: int,
                             partition_size: int = 0) -> int:
    return int(lib.pkv_attention_plan_words(S, Hkv, B, max_blocks, max_context_len,
                                            partition_size))


def pkv_attention_plan(context_lens, Hkv: int, B: int, max_blocks: int, max_context_len: int,
                       partition_size: int = 0):
    """Host plan for a batch from its HOST lengths: (int32 words, n_items, n_merge)."""
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    S = lens.shape[0]
    cap = pkv_attention_plan_words(S, Hkv, B, max_blocks, max_context_len, partition_size)
    words = np.zeros(max(cap, 4), np.int32)
    n_items, n_merge = _i32(), _i32()
    _check(lib.pkv_attention_plan(_np_ptr(lens, ctypes.c_int32), S, Hkv, B, max_blocks,
                                  max_context_len, partition_size, _np_ptr(words, ctypes.c_int32),
                                  words.shape[0], ctypes.byref(n_items), ctypes.byref(n_merge)),
           "pkv_attention_plan")
    used = 4 * n_items.value + n_merge.value
    return words[:used].copy(), n_items.value, n_merge.value


def make_plan(context_lens, Hkv: int, B: int, max_blocks: int, max_context_len: int,
              partition_size: int = 0, device="cuda") -> Plan:
    """pkv_attention_plan, then the copy to the device."""
    words, n_items, n_merge = pkv_attention_plan(context_lens, Hkv, B, max_blocks,
                                                 max_context_len, partition_size)
    dev = torch.from_numpy(words if words.size else np.zeros(4, np.int32)).to(device)
    return Plan(dev, n_items, n_merge)


def _plan_args(plan):
    if plan is None:
        return None, 0, 0
    if not isinstance(plan, Plan):
        raise TypeError("plan must be a Plan (see make_plan)")
    return _dev(plan.words, "plan"), plan.n_items, plan.n_merge


def _attention_args(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                    scale, partition_size, plan, workspace, shared_kv, new_key, new_value,
                    k_scale=None, v_scale=None):
    N, Hkv, D, B = _pool_geometry(k_pool, v_pool)
    S, Hq = q.shape[0], q.shape[1]
    nk = nv = None
    if (new_key is None) != (new_value is None):
        raise ValueError("new_key and new_value go together")
    if new_key is not None:
        for t, name in ((new_key, "new_key"), (new_value, "new_value")):
            if tuple(t.shape) != (S, Hkv, D) or t.dtype != _row_dtype(k_pool):
                raise ValueError(f"{name} must be [S, Hkv, D] in the pool dtype "
                                 f"(bf16 for fp8 pools)")
        nk, nv = _dev(new_key, "new_key"), _dev(new_value, "new_value")
    if tuple(q.shape) != (S, Hq, D) or q.dtype != _row_dtype(k_pool):
        raise ValueError("q must be [S, Hq, D] in the pool dtype (bf16 for fp8 pools)")
    if out.dtype != torch.float32 or tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must be float32 [S, Hq, D]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [S, max_blocks]")
    if context_lens.dtype != torch.int32 or tuple(context_lens.shape) != (S,):
        raise ValueError("context_lens must be int32 [S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    return (_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
            nk, nv, _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), S, Hq,
            Hkv, D,
            B, block_tables.shape[1], N, int(max_context_len), float(scale), int(partition_size),
            *_plan_args(plan), ws_ptr, ws_bytes, _dtype_code(k_pool),
            PKV_ATTN_SHARED_KV if shared_kv else 0, *_scales(k_pool, k_scale, v_scale, Hkv))


def pkv_paged_attention_decode(out, q, k_pool, v_pool, block_tables, context_lens,
                               max_context_len: int, scale: float | None = None,
                               partition_size: int = 0, workspace=None, stream=None,
                               shared_kv: bool = False, plan: Plan | None = None,
                               new_key=None, new_value=None, k_scale=None,
                               v_scale=None) -> None:
    """out[s, h] = softmax(q[s, h] K_s^T * scale) V_s through the block tables.

    out fp32 [S, Hq, D]; q [S, Hq, D] in the pool dtype; block_tables int32
    [S, max_blocks]; context_lens int32 [S].  `workspace` (a uint8 device tensor)
    is needed when max_context_len exceeds one partition.  `shared_kv` sets
    PKV_ATTN_SHARED_KV (the batch shares blocks; a load-policy hint only).
    `plan` (make_plan) runs exactly the batch's work items.  `new_key` /
    `new_value` ([S, Hkv, D]; bf16 for fp8 pools, encoded with the scales) append
    each sequence's token of this step (its position context_lens[s]-1) into the
    pools in the same launch.  fp8 pools
    (uint8 / float8_e4m3fn) take bf16 q and the per-head k_scale / v_scale
    (float32 [Hkv] device tensors)."""
    args = _attention_args(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                           scale, partition_size, plan, workspace, shared_kv, new_key, new_value,
                           k_scale, v_scale)
    _check(lib.pkv_paged_attention_decode(*args, _stream(stream)), "pkv_paged_attention_decode")


def pkv_paged_attention_main(out, q, k_pool, v_pool, block_tables, context_lens,
                             max_context_len: int, scale: float | None = None,
                             partition_size: int = 0, workspace=None, stream=None,
                             shared_kv: bool = False, plan: Plan | None = None,
                             new_key=None, new_value=None, k_scale=None,
                             v_scale=None) -> None:
    """The main launch of pkv_paged_attention_decode alone (same arguments)."""
    args = _attention_args(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                           scale, partition_size, plan, workspace, shared_kv, new_key, new_value,
                           k_scale, v_scale)
    _check(lib.pkv_paged_attention_main(*args, _stream(stream)), "pkv_paged_attention_main")


def pkv_paged_attention_decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens,
                                       max_context_len: int, scale: float | None = None,
                                       partition_size: int = 0, stream=None,
                                       shared_kv: bool = False, plan: Plan | None = None,
                                       new_key=None, new_value=None, k_scale=None,
                                       v_scale=None) -> None:
    """pkv_paged_attention_decode without a workspace: the library's static
    per-GPU scratch holds the partials (PKV_ENOSCRATCH when the call needs more
    than PKV_SCRATCH_BYTES).  Calls that overlap in time on one GPU race."""
    args = _attention_args(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                           scale, partition_size, plan, None, shared_kv, new_key, new_value,
                           k_scale, v_scale)
    # the same arguments without workspace and workspace_bytes
    args = args[:21] + args[23:]
    _check(lib.pkv_paged_attention_decode_noalloc(*args, _stream(stream)),
           "pkv_paged_attention_decode_noalloc")


def pkv_paged_attention_reduce(out, context_lens, Hkv: int, B: int, max_blocks: int,
                               max_context_len: int, partition_size: int = 0, workspace=None,
                               stream=None, plan: Plan | None = None) -> None:
    """The partition merge of pkv_paged_attention_decode alone; the arguments
    repeat those of the preceding pkv_paged_attention_main call."""
    S, Hq, D = out.shape
    if out.dtype != torch.float32:
        raise ValueError("out must be float32 [S, Hq, D]")
    if context_lens.dtype != torch.int32 or tuple(context_lens.shape) != (S,):
        raise ValueError("context_lens must be int32 [S]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_attention_reduce(_dev(out, "out"), _dev(context_lens, "context_lens"),
                                          S, Hq, int(Hkv), D, int(B), int(max_blocks),
                                          int(max_context_len), int(partition_size),
                                          *_plan_args(plan), ws_ptr, ws_bytes, _stream(stream)),
           "pkv_paged_attention_reduce")


reshape_and_cache = pkv_reshape_and_cache
copy_blocks = pkv_copy_blocks
swap_blocks = pkv_swap_blocks
paged_attention_prefill = pkv_paged_attention_prefill
attention_workspace_bytes = pkv_attention_workspace_bytes
paged_attention_decode = pkv_paged_attention_decode
paged_attention_main = pkv_paged_attention_main
paged_attention_reduce = pkv_paged_attention_reduce
paged_attention_decode_noalloc = pkv_paged_attention_decode_noalloc
attention_plan = pkv_attention_plan
attention_plan_words = pkv_attention_plan_words
