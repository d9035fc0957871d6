"""Reference cache writes: reshape_and_cache and copy_blocks (bit copies).

reshape_and_cache: each newly generated token's K/V vectors are added to its
sequence's cache ("PagedAttention: The vLLM Paper", "Background and
Motivation"), into the block allocated for it ("PagedAttention and Continuous
Batching", "Pages, from operating systems": new blocks are allocated as tokens
are generated).  A token's slot is physical_block * B + offset; a negative slot
means "no token here" (padding) and is skipped.

copy_blocks: a shared block is copied only when one sequence is about to
modify it, like copy-on-write after an OS fork ("Pages, from operating
systems"; "The Core Idea", OS-paging analogy table).  The whole block (all
heads, all slots, K and V) is copied.

Both operate on raw element arrays (float32, or bf16 as uint16), so every copy
is a bit copy and NaN payloads survive unchanged.
"""
from __future__ import annotations

import numpy as np

from oracle import fp8


def _f32(a):
    """bf16 bit patterns (uint16) or fp32 -> fp32, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def reshape_and_cache(k_pool, v_pool, key, value, slot_mapping, k_scale=None, v_scale=None):
    """Return new (k_pool, v_pool) with token i written to slot_mapping[i].

    key/value: [T, Hkv, D]; k_pool [N, Hkv, D/x, B, x]; v_pool [N, Hkv, D, B].
    fp8 pools (uint8): key/value (bf16 bits or fp32) are quantized to E4M3
    with the per-KV-head scales first (oracle/fp8.py)."""
    N, Hkv, Dx, B, x = k_pool.shape
    if k_pool.dtype == np.uint8:
        key = fp8.quantize(_f32(key), k_scale, head_axis=1)
        value = fp8.quantize(_f32(value), v_scale, head_axis=1)
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        slot = int(slot)
        if slot < 0:
            continue
        pb, off = divmod(slot, B)
        k_out[pb, :, :, off, :] = key[i].reshape(Hkv, Dx, x)
        v_out[pb, :, :, off] = value[i]
    return k_out, v_out


def copy_blocks(k_pool, v_pool, pairs):
    """Return new pools with block dst := block src for every (src, dst).
    Sources are read from the pools as given (no dst is also a src)."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_out[int(dst)] = k_pool[int(src)]
        v_out[int(dst)] = v_pool[int(src)]
    return k_out, v_out
