"""Pins for the reference attention (CPU only).

Paging must not change the attention result: paged == contiguous library
attention (torch SDPA in fp64), == a scalar brute-force loop, plus closed forms
(L=1, identical keys, zero query), the GQA head map, NaN in unused slots, and
the log-sum-exp split identity."""
import math

import numpy as np
import pytest
import torch

from oracle.attention import (attention, combine_partials, gather_kv, paged_attention_decode,
                              partition_partials, to_f64, valid_slot_mask)
from oracle.block_manager import BlockManager
from oracle.cache_ops import reshape_and_cache
from workloads import normal, pool_shapes


def _bits(x32):
    """fp32 -> bf16 bit patterns by truncation (exact for the values used)."""
    return (np.asarray(x32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_bf16_widening_closed_form():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001], np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, (2 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** -133]
    got = to_f64(bits)
    assert got.tolist() == want
    assert math.copysign(1, got[4]) == -1


def _paged_setup(rng, lens, Hkv, D, B, dtype, extra=3):
    """Build a pool holding contiguous per-sequence K/V through the reference
    block manager + reshape_and_cache.  Returns the pool, tables, and the
    contiguous arrays each sequence wrote."""
    need = sum(-(-L // B) for L in lens)
    N = need + extra
    bm = BlockManager(N, B, rng.permutation(N))
    ks, vs = pool_shapes(N, Hkv, D, B, dtype)
    k_pool = normal(rng, ks, dtype)
    v_pool = normal(rng, vs, dtype)
    Ks, Vs = [], []
    for s, L in enumerate(lens):
        bm.add_seq(s, 0)
        K = normal(rng, (L, Hkv, D), dtype)
        V = normal(rng, (L, Hkv, D), dtype)
        slots = [bm.append_slot(s)[0] for _ in range(L)]
        k_pool, v_pool = reshape_and_cache(k_pool, v_pool, K, V, slots)
        Ks.append(K)
        Vs.append(V)
    maxb = max(-(-L // B) for L in lens)
    tables, clens = bm.fill_batch(range(len(lens)), maxb)
    return k_pool, v_pool, np.array(tables), np.array(clens), Ks, Vs, N


@pytest.mark.parametrize("dtype,B,G", [("f32", 16, 1), ("bf16", 16, 4), ("bf16", 32, 8),
                                       ("bf16", 4, 2)])
def test_paged_equals_contiguous_sdpa(dtype, B, G):
    rng = np.random.default_rng(7)
    Hkv, D = 2, 32
    Hq = Hkv * G
    lens = [1, B - 1, B, B + 1, 3 * B + 5, 70]
    k_pool, v_pool, tables, clens, Ks, Vs, _ = _paged_setup(rng, lens, Hkv, D, B, dtype)
    q = normal(rng, (len(lens), Hq, D), dtype)
    scale = 1.0 / math.sqrt(D)
    out = paged_attention_decode(q, k_pool, v_pool, tables, clens, scale)
    for s, L in enumerate(lens):
        qs = torch.from_numpy(to_f64(q[s])).view(Hkv, G, 1, D)
        K = torch.from_numpy(to_f64(Ks[s])).permute(1, 0, 2).reshape(Hkv, 1, L, D)
        V = torch.from_numpy(to_f64(Vs[s])).permute(1, 0, 2).reshape(Hkv, 1, L, D)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qs, K.expand(Hkv, G, L, D), V.expand(Hkv, G, L, D), scale=scale)
        np.testing.assert_allclose(out[s], ref.reshape(Hq, D).numpy(), rtol=0, atol=1e-12)


def test_brute_force_scalar_loops():
    rng = np.random.default_rng(11)
    Hkv, G, D, B = 2, 2, 4, 2
    lens = [1, 3, 5]
    k_pool, v_pool, tables, clens, Ks, Vs, _ = _paged_setup(rng, lens, Hkv, D, B, "f32")
    q = normal(rng, (len(lens), Hkv * G, D), "f32")
    scale = 0.5
    out = paged_attention_decode(q, k_pool, v_pool, tables, clens, scale)
    for s, L in enumerate(lens):
        for h in range(Hkv * G):
            g = h // G
            z = []
            for t in range(L):
                acc = 0.0
                for d in range(D):
                    acc += float(q[s, h, d]) * float(Ks[s][t, g, d])
                z.append(acc * scale)
            mx = max(z)
            w = [math.exp(v - mx) for v in z]
            tot = sum(w)
            for d in range(D):
                ref = sum(w[t] * float(Vs[s][t, g, d]) for t in range(L)) / tot
                assert abs(out[s, h, d] - ref) <= 1e-13


def test_closed_forms():
    rng = np.random.default_rng(5)
    D = 16
    V = rng.standard_normal((9, D))
    q = rng.standard_normal(D)
    # L = 1: the output is the single value row, exactly
    assert np.array_equal(attention(q, rng.standard_normal((1, D)), V[:1], 0.25), V[0])
    # identical keys, or a zero query: uniform weights -> mean of V
    K = np.tile(rng.standard_normal(D), (9, 1))
    np.testing.assert_allclose(attention(q, K, V, 0.25), V.mean(0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(attention(np.zeros(D), rng.standard_normal((9, D)), V, 0.25),
                               V.mean(0), rtol=0, atol=1e-14)
    # one dominant key selects its value row
    K = np.zeros((9, D))
    K[4] = 1000.0 * q / np.linalg.norm(q)
    np.testing.assert_allclose(attention(q, K, V, 1.0), V[4], rtol=0, atol=1e-12)


def test_gqa_head_map():
    """Query head h reads KV head h // G: perturbing KV head g changes exactly
    the outputs of heads g*G .. g*G+G-1."""
    rng = np.random.default_rng(3)
    Hkv, G, D, B = 4, 2, 8, 4
    lens = [6, 9]
    k_pool, v_pool, tables, clens, _, _, _ = _paged_setup(rng, lens, Hkv, D, B, "f32")
    q = normal(rng, (2, Hkv * G, D), "f32")
    base = paged_attention_decode(q, k_pool, v_pool, tables, clens)
    for g in range(Hkv):
        v2 = v_pool.copy()
        v2[:, g] += 1.0
        out = paged_attention_decode(q, k_pool, v2, tables, clens)
        changed = np.abs(out - base).max(axis=(0, 2)) > 0.5
        assert changed.tolist() == [h // G == g for h in range(Hkv * G)]


def test_physical_placement_is_invisible():
    """The same tokens in a shuffled pool give a bit-identical result (same
    gathered arrays, same summation order)."""
    rng = np.random.default_rng(9)
    Hkv, D, B = 2, 16, 4
    lens = [5, 13, 8]
    k_pool, v_pool, tables, clens, _, _, N = _paged_setup(rng, lens, Hkv, D, B, "bf16")
    q = normal(rng, (3, Hkv, D), "bf16")
    out = paged_attention_decode(q, k_pool, v_pool, tables, clens)
    perm = rng.permutation(N)                      # physical block b moves to perm[b]
    k2 = np.empty_like(k_pool)
    v2 = np.empty_like(v_pool)
    k2[perm] = k_pool
    v2[perm] = v_pool
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    out2 = paged_attention_decode(q, k2, v2, t2, clens)
    assert np.array_equal(out, out2)


def test_unused_slots_do_not_leak():
    """NaN in every slot that holds no token leaves the output finite and equal."""
    rng = np.random.default_rng(13)
    Hkv, D, B = 2, 16, 16
    lens = [1, 15, 16, 17, 40]
    k_pool, v_pool, tables, clens, _, _, N = _paged_setup(rng, lens, Hkv, D, B, "bf16")
    q = normal(rng, (len(lens), Hkv, D), "bf16")
    out = paged_attention_decode(q, k_pool, v_pool, tables, clens)
    mask = valid_slot_mask(tables, clens, N, B)
    k2, v2 = k_pool.copy(), v_pool.copy()
    nan = np.uint16(0x7FC1)
    for b in range(N):
        for o in range(B):
            if not mask[b, o]:
                k2[b, :, :, o, :] = nan
                v2[b, :, :, o] = nan
    out2 = paged_attention_decode(q, k2, v2, tables, clens)
    assert np.isfinite(out2).all() and np.array_equal(out, out2)


@pytest.mark.parametrize("L,P", [(1, 512), (100, 16), (512, 512), (513, 512), (4000, 512),
                                 (33, 32), (4096, 64)])
def test_split_k_identity(L, P):
    rng = np.random.default_rng(L + P)
    D = 32
    K = rng.standard_normal((L, D)) * 3
    V = rng.standard_normal((L, D))
    q = rng.standard_normal(D)
    whole = attention(q, K, V, 1 / math.sqrt(D))
    split = combine_partials(partition_partials(q, K, V, 1 / math.sqrt(D), P))
    np.testing.assert_allclose(split, whole, rtol=0, atol=1e-12)


def test_gather_reads_only_valid_tokens():
    rng = np.random.default_rng(2)
    Hkv, D, B = 1, 8, 4
    k_pool, v_pool, tables, clens, Ks, Vs, _ = _paged_setup(rng, [7], Hkv, D, B, "f32")
    K, V = gather_kv(k_pool, v_pool, tables[0], 7, 0)
    assert np.array_equal(K, Ks[0][:, 0].astype(np.float64))
    assert np.array_equal(V, Vs[0][:, 0].astype(np.float64))
