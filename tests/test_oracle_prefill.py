"""Pins for the multi-token (chunked prefill / prefix-hit) reference attention
(CPU only).

What fixes the result: each new token attends causally over itself and every
earlier token of its sequence ("Background and Motivation"), and paging does
not change attention.  Pinned against: the decode reference (one query per
sequence is decode), a library attention (torch SDPA in fp64 with an explicit
bottom-right causal mask over contiguous K/V), scalar brute force, the
chunking identity (a prompt attended in one chunk or in several gives the same
rows: what chunked prefill relies on, "Impact and Follow-Ups"), and physical
placement (a prefix shared through the block table gives the same rows as a
private copy: what prefix caching relies on)."""
import math

import numpy as np
import pytest
import torch

from oracle.attention import (paged_attention_decode, paged_attention_prefill, query_starts,
                              to_f64)
from oracle.block_manager import BlockManager
from oracle.cache_ops import reshape_and_cache
from tests.test_oracle_attention import _paged_setup
from workloads import normal, pool_shapes


def test_one_query_per_sequence_is_decode():
    rng = np.random.default_rng(21)
    Hkv, G, D, B = 2, 4, 32, 16
    lens = [1, 15, 16, 17, 70]
    k_pool, v_pool, tables, clens, _, _, _ = _paged_setup(rng, lens, Hkv, D, B, "bf16")
    q = normal(rng, (len(lens), Hkv * G, D), "bf16")
    got = paged_attention_prefill(q, k_pool, v_pool, tables, clens, [1] * len(lens))
    want = paged_attention_decode(q, k_pool, v_pool, tables, clens)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype,B,G", [("bf16", 16, 4), ("bf16", 32, 1), ("f32", 4, 2),
                                       ("bf16", 16, 8)])
def test_prefill_equals_masked_sdpa(dtype, B, G):
    rng = np.random.default_rng(23)
    Hkv, D = 2, 32
    Hq = Hkv * G
    lens = [1, 9, 16, 33, 70]
    qlens = [1, 9, 5, 16, 70]              # a whole prompt, a chunk, a prefix hit ...
    k_pool, v_pool, tables, clens, Ks, Vs, _ = _paged_setup(rng, lens, Hkv, D, B, dtype)
    T = sum(qlens)
    q = normal(rng, (T, Hq, D), dtype)
    scale = 1.0 / math.sqrt(D)
    out = paged_attention_prefill(q, k_pool, v_pool, tables, clens, qlens, scale)
    starts = query_starts(qlens)
    for s, (L, Q) in enumerate(zip(lens, qlens)):
        qs = torch.from_numpy(to_f64(q[starts[s]:starts[s + 1]]))          # [Q, Hq, D]
        qs = qs.permute(1, 0, 2).reshape(Hkv, G, Q, D)
        K = torch.from_numpy(to_f64(Ks[s])).permute(1, 0, 2).reshape(Hkv, 1, L, D)
        V = torch.from_numpy(to_f64(Vs[s])).permute(1, 0, 2).reshape(Hkv, 1, L, D)
        pos = torch.arange(L - Q, L).view(Q, 1)
        mask = torch.arange(L).view(1, L) <= pos                            # bottom-right causal
        ref = torch.nn.functional.scaled_dot_product_attention(
            qs, K.expand(Hkv, G, L, D), V.expand(Hkv, G, L, D), attn_mask=mask, scale=scale)
        ref = ref.reshape(Hq, Q, D).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[starts[s]:starts[s + 1]], ref, rtol=0, atol=1e-12)


def test_brute_force_scalar_loops():
    rng = np.random.default_rng(29)
    Hkv, G, D, B = 1, 2, 4, 2
    lens, qlens = [4, 5], [3, 2]
    k_pool, v_pool, tables, clens, Ks, Vs, _ = _paged_setup(rng, lens, Hkv, D, B, "f32")
    q = normal(rng, (sum(qlens), Hkv * G, D), "f32")
    scale = 0.7
    out = paged_attention_prefill(q, k_pool, v_pool, tables, clens, qlens, scale)
    row = 0
    for s, (L, Q) in enumerate(zip(lens, qlens)):
        for i in range(Q):
            p = L - Q + i
            for h in range(Hkv * G):
                z = [sum(float(q[row, h, d]) * float(Ks[s][t, h // G, d]) for d in range(D)) * scale
                     for t in range(p + 1)]
                w = [math.exp(v - max(z)) for v in z]
                for d in range(D):
                    ref = sum(w[t] * float(Vs[s][t, h // G, d]) for t in range(p + 1)) / sum(w)
                    assert abs(out[row, h, d] - ref) <= 1e-13
            row += 1


def test_chunks_give_the_rows_of_one_pass():
    """Attending a 70-token prompt as one chunk, or as chunks of 16 + 30 + 24
    over the growing cache, gives the same rows bit for bit."""
    rng = np.random.default_rng(31)
    Hkv, G, D, B = 2, 2, 16, 16
    L = 70
    k_pool, v_pool, tables, clens, _, _, _ = _paged_setup(rng, [L], Hkv, D, B, "bf16")
    q = normal(rng, (L, Hkv * G, D), "bf16")
    whole = paged_attention_prefill(q, k_pool, v_pool, tables, [L], [L])
    done = 0
    for chunk in (16, 30, 24):
        part = paged_attention_prefill(q[done:done + chunk], k_pool, v_pool, tables,
                                       [done + chunk], [chunk])
        assert np.array_equal(part, whole[done:done + chunk])
        done += chunk


def test_shared_prefix_blocks_are_invisible():
    """Two requests whose prompts share a 32-token prefix: one reads the prefix
    through the other's blocks (a prefix-cache hit), one through a private
    copy; their suffix rows agree exactly."""
    rng = np.random.default_rng(37)
    Hkv, G, D, B = 2, 4, 32, 16
    prefix, suffix = 32, 13
    N = 12
    bm = BlockManager(N, B, rng.permutation(N))
    ks, vs = pool_shapes(N, Hkv, D, B, "bf16")
    k_pool, v_pool = normal(rng, ks, "bf16"), normal(rng, vs, "bf16")
    Kp, Vp = normal(rng, (prefix, Hkv, D), "bf16"), normal(rng, (prefix, Hkv, D), "bf16")
    Ks, Vs = normal(rng, (suffix, Hkv, D), "bf16"), normal(rng, (suffix, Hkv, D), "bf16")
    # request 0: writes prefix + suffix into its own blocks
    bm.add_seq(0, prefix + suffix)
    k_pool, v_pool = reshape_and_cache(k_pool, v_pool, np.concatenate([Kp, Ks]),
                                       np.concatenate([Vp, Vs]), _slots(bm, 0, 0, prefix + suffix))
    # request 1: shares request 0's two prefix blocks, writes only its suffix
    bm.add_seq(1, 0)
    bm.tables[1] = list(bm.tables[0][:prefix // B])
    for b in bm.tables[1]:
        bm.ref[b] += 1
    bm.lens[1] = prefix
    sl = [bm.append_slot(1)[0] for _ in range(suffix)]
    k_pool, v_pool = reshape_and_cache(k_pool, v_pool, Ks, Vs, sl)
    assert bm.tables[1][:2] == bm.tables[0][:2] and bm.tables[1][2] != bm.tables[0][2]
    tables, clens = bm.fill_batch([0, 1], 3)
    q = normal(rng, (suffix, Hkv * G, D), "bf16")
    out = paged_attention_prefill(np.concatenate([q, q]), k_pool, v_pool, np.array(tables),
                                  clens, [suffix, suffix])
    assert np.array_equal(out[:suffix], out[suffix:])


def _slots(bm, sid, start, count):
    t = bm.tables[sid]
    return [t[i // bm.B] * bm.B + i % bm.B for i in range(start, start + count)]


def test_rows_subset_and_bad_lengths():
    rng = np.random.default_rng(41)
    k_pool, v_pool, tables, clens, _, _, _ = _paged_setup(rng, [20, 9], 1, 16, 16, "f32")
    q = normal(rng, (7, 2, 16), "f32")
    full = paged_attention_prefill(q, k_pool, v_pool, tables, clens, [4, 3])
    some = paged_attention_prefill(q, k_pool, v_pool, tables, clens, [4, 3], rows=[(5, 1)])
    assert np.array_equal(some[5, 1], full[5, 1]) and np.isnan(some[0]).all()
    with pytest.raises(ValueError):
        paged_attention_prefill(q, k_pool, v_pool, tables, clens, [4, 4])    # rows != T
    with pytest.raises(ValueError):
        paged_attention_prefill(q[:2], k_pool, v_pool, tables, [1, 9], [2, 0])   # Q > L
