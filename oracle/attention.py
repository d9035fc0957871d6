"""fp64 reference for PagedAttention decode.

What is computed (PagedAttention: The vLLM Paper, "Background and Motivation":
each new token attends over all previous tokens; "The Core Idea": attention is
computed through block-table indirection over non-contiguous blocks;
vLLM: PagedAttention and continuous batching, "Direct answer": PagedAttention
follows the logical->physical block mapping while computing attention).  Paging
changes where K/V live, not the attention result, so the oracle gathers each
sequence's tokens back into contiguous arrays and applies the textbook
definition softmax(q K^T * scale) V in fp64.

Readings where the pages are silent:
  * pool layout (the library's ABI): K pool [N, Hkv, D/x, B, x] and V pool
    [N, Hkv, D, B], x = elements per 16 bytes; token at logical position t of a
    sequence lives in physical block table[t // B], slot t % B;
  * L_s counts every cached token including the one written this step;
  * query head h reads KV head h // (Hq / Hkv) (consecutive heads share);
  * bf16 values are held as raw uint16 bit patterns and widened exactly;
  * an fp8 pool (uint8 E4M3 codes, oracle/fp8.py) holds K and V divided by a
    per-KV-head scale: the value of a code times its head's scale, exact in
    fp64, is what attention uses.
"""
from __future__ import annotations

import numpy as np

from oracle import fp8


def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening: float32 -> fp64, or bf16 bit patterns (uint16) -> fp64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.float32 or a.dtype == np.float64:
        return a.astype(np.float64)
    raise TypeError(f"unsupported element type {a.dtype}")


def _widen(a: np.ndarray, scale) -> np.ndarray:
    if a.dtype == np.uint8:
        return fp8.DECODE[a] * float(scale)
    return to_f64(a)


def gather_kv(k_pool, v_pool, table, L: int, g: int, k_scale=None, v_scale=None):
    """Contiguous K, V [L, D] (fp64) of one sequence and KV head `g` (fp8 pools
    are dequantized with the head's scales).

    Logical block j of the sequence is physical block table[j]; it holds
    tokens j*B .. j*B+B-1, of which only the first L - j*B are valid when it is
    the last block (only the last block may be partially filled)."""
    N, Hkv, Dx, B, x = k_pool.shape
    D = Dx * x
    K = np.empty((L, D), dtype=np.float64)
    V = np.empty((L, D), dtype=np.float64)
    nblocks = -(-L // B)
    for j in range(nblocks):
        pb = int(table[j])
        n = min(B, L - j * B)
        # K block [D/x, B, x] -> tokens x dims
        kb = k_pool[pb, g, :, :n, :]                 # [D/x, n, x]
        ks = None if k_scale is None else k_scale[g]
        vs = None if v_scale is None else v_scale[g]
        K[j * B:j * B + n] = _widen(np.transpose(kb, (1, 0, 2)).reshape(n, D), ks)
        vb = v_pool[pb, g, :, :n]                    # [D, n]
        V[j * B:j * B + n] = _widen(vb.T, vs)
    return K, V


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V for one query vector, fp64, max-subtracted."""
    z = (K @ q) * scale
    z = z - z.max()
    p = np.exp(z)
    return (p @ V) / p.sum()


def paged_attention_decode(q, k_pool, v_pool, block_tables, context_lens, scale=None,
                           rows=None, k_scale=None, v_scale=None):
    """Decode attention for every (sequence, query head), or only `rows`
    (a list of (s, h) pairs).  Returns fp64 [S, Hq, D] (unsampled rows are NaN)."""
    S, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((S, Hq, D), np.nan)
    want = None if rows is None else {}
    if rows is not None:
        for s, h in rows:
            want.setdefault(int(s), set()).add(int(h))
    qf = to_f64(q)
    for s in range(S):
        if want is not None and s not in want:
            continue
        L = int(context_lens[s])
        for g in range(Hkv):
            heads = [h for h in range(g * G, (g + 1) * G) if want is None or h in want[s]]
            if not heads:
                continue
            K, V = gather_kv(k_pool, v_pool, block_tables[s], L, g, k_scale, v_scale)
            for h in heads:
                out[s, h] = attention(qf[s, h], K, V, scale)
    return out


def query_starts(query_lens) -> np.ndarray:
    """Offsets of each sequence's first query row in the packed query array."""
    starts = np.zeros(len(query_lens) + 1, dtype=np.int64)
    np.cumsum(np.asarray(query_lens, dtype=np.int64), out=starts[1:])
    return starts


def paged_attention_prefill(q, k_pool, v_pool, block_tables, context_lens, query_lens,
                            scale=None, rows=None, k_scale=None, v_scale=None):
    """Attention of several new tokens per sequence over the paged cache
    (chunked prefill, and the uncached rest of a prompt after a prefix-cache
    hit: PagedAttention: The vLLM Paper, "Impact and Follow-Ups").

    Sequence s holds L_s = context_lens[s] cached tokens, the last Q_s =
    query_lens[s] of which are this call's queries (their K/V are already in
    the cache).  The query at position p = L_s - Q_s + i attends to tokens
    0..p: each token attends over itself and every earlier token ("Background
    and Motivation").  q packs the sequences' query rows [T, Hq, D], T = sum
    Q_s, sequence by sequence in batch order.  Returns fp64 [T, Hq, D]; with
    `rows` (a list of (packed row, head) pairs) only those are computed and the
    rest are NaN."""
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    starts = query_starts(query_lens)
    if starts[-1] != T:
        raise ValueError("query rows must total sum(query_lens)")
    out = np.full((T, Hq, D), np.nan)
    want = None
    if rows is not None:
        want = {}
        for t, h in rows:
            want.setdefault(int(t), set()).add(int(h))
    qf = to_f64(q)
    for s in range(len(query_lens)):
        L, Q = int(context_lens[s]), int(query_lens[s])
        if not 0 <= Q <= L:
            raise ValueError("each sequence needs 0 <= query_lens <= context_lens")
        for g in range(Hkv):
            K = V = None
            for i in range(Q):
                t = int(starts[s]) + i
                heads = [h for h in range(g * G, (g + 1) * G)
                         if want is None or h in want.get(t, ())]
                if not heads:
                    continue
                if K is None:
                    K, V = gather_kv(k_pool, v_pool, block_tables[s], L, g, k_scale, v_scale)
                p = L - Q + i
                for h in heads:
                    out[t, h] = attention(qf[t, h], K[:p + 1], V[:p + 1], scale)
    return out


def partition_partials(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, P: int):
    """Split the context into partitions of P tokens and return, per partition,
    (m, l, acc): the max score, the sum of exp(score - m) and the unnormalised
    exp-weighted sum of V rows.  This split is not on the pages; it is the
    standard way to cut one long context across many workgroups."""
    L = K.shape[0]
    parts = []
    for start in range(0, L, P):
        z = (K[start:start + P] @ q) * scale
        m = z.max()
        p = np.exp(z - m)
        parts.append((m, p.sum(), p @ V[start:start + P]))
    return parts


def combine_partials(parts) -> np.ndarray:
    """Log-sum-exp combine: rescale each partition to the global max M, then
    divide the summed numerators by the summed denominators."""
    M = max(m for m, _, _ in parts)
    num = sum(np.exp(m - M) * acc for m, _, acc in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    return num / den


def valid_slot_mask(block_tables, context_lens, num_blocks: int, B: int) -> np.ndarray:
    """bool [N, B]: which (physical block, slot) pairs hold a token of some
    sequence.  Everything else is free or past a sequence's end."""
    mask = np.zeros((num_blocks, B), dtype=bool)
    for table, L in zip(block_tables, context_lens):
        L = int(L)
        for t in range(L):
            mask[int(table[t // B]), t % B] = True
    return mask
