"""Pins for the reference cache writes (CPU only)."""
import math

import numpy as np

from oracle.attention import attention, gather_kv, paged_attention_decode, to_f64
from oracle.block_manager import BlockManager
from oracle.cache_ops import copy_blocks, reshape_and_cache
from workloads import normal, pool_shapes


def test_written_token_gathers_back_bit_exact():
    rng = np.random.default_rng(0)
    N, Hkv, D, B = 6, 2, 16, 4
    ks, vs = pool_shapes(N, Hkv, D, B, "bf16")
    kp, vp = normal(rng, ks, "bf16"), normal(rng, vs, "bf16")
    key = normal(rng, (3, Hkv, D), "bf16")
    val = normal(rng, (3, Hkv, D), "bf16")
    key[1, 0, 3] = 0x7FC5          # a NaN payload must survive as bits
    slots = [4 * 2 + 1, -1, 5 * 4 + 3]
    kp2, vp2 = reshape_and_cache(kp, vp, key, val, slots)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        pb, off = divmod(slot, B)
        for g in range(Hkv):
            table = [pb]
            K, V = gather_kv(kp2, vp2, table, off + 1, g)
            assert np.array_equal(K[off], to_f64(key[i, g]))
            assert np.array_equal(V[off], to_f64(val[i, g]))
    # a skipped token changes nothing; only the two written slots differ
    changed_k = np.argwhere((kp2 != kp).any(axis=(1, 2, 4)))
    changed_v = np.argwhere((vp2 != vp).any(axis=(1, 2)))
    assert sorted(map(tuple, changed_k)) == [(2, 1), (5, 3)]
    assert sorted(map(tuple, changed_v)) == [(2, 1), (5, 3)]
    # the NaN slot was written bit for bit (token 1 was skipped, so write it now)
    kp3, _ = reshape_and_cache(kp, vp, key, val, [-1, 0, -1])
    assert kp3.view(np.uint16)[0, 0, 0, 0, 3] == 0x7FC5


def test_copy_blocks_copies_whole_blocks():
    rng = np.random.default_rng(1)
    N, Hkv, D, B = 8, 2, 8, 4
    ks, vs = pool_shapes(N, Hkv, D, B, "f32")
    kp, vp = normal(rng, ks, "f32"), normal(rng, vs, "f32")
    kp[3, 1, 0, 2, 1] = np.float32("nan")
    kp2, vp2 = copy_blocks(kp, vp, [(3, 6), (1, 0)])
    assert kp2[6].tobytes() == kp[3].tobytes() and vp2[6].tobytes() == vp[3].tobytes()
    assert kp2[0].tobytes() == kp[1].tobytes() and vp2[0].tobytes() == vp[1].tobytes()
    for b in (1, 2, 3, 4, 5, 7):
        assert kp2[b].tobytes() == kp[b].tobytes() and vp2[b].tobytes() == vp[b].tobytes()


def test_copy_on_write_step_semantics():
    """fork -> append (CoW) -> copy_blocks -> reshape_and_cache: the writer sees
    its own tokens, and every other sharer's attention is unchanged."""
    rng = np.random.default_rng(4)
    Hkv, D, B, G = 2, 16, 16, 2
    N = 12
    bm = BlockManager(N, B, rng.permutation(N))
    ks, vs = pool_shapes(N, Hkv, D, B, "bf16")
    kp, vp = normal(rng, ks, "bf16"), normal(rng, vs, "bf16")
    P = 21                                                   # prompt: 1 full + 1 partial block
    Kp, Vp = normal(rng, (P, Hkv, D), "bf16"), normal(rng, (P, Hkv, D), "bf16")
    bm.add_seq(0, 0)
    kp, vp = reshape_and_cache(kp, vp, Kp, Vp, [bm.append_slot(0)[0] for _ in range(P)])
    for c in (1, 2):
        bm.fork(0, c)
    q = normal(rng, (3, Hkv * G, D), "bf16")
    tables, lens = bm.fill_batch([0, 1, 2], 2)
    before = paged_attention_decode(q, kp, vp, np.array(tables), np.array(lens))
    # sequence 1 generates a token: its shared partial block must be copied first
    slot, src, dst = bm.append_slot(1)
    assert src == tables[1][1] and dst >= 0
    kn, vn = normal(rng, (1, Hkv, D), "bf16"), normal(rng, (1, Hkv, D), "bf16")
    kp, vp = copy_blocks(kp, vp, [(src, dst)])
    kp, vp = reshape_and_cache(kp, vp, kn, vn, [slot])
    tables, lens = bm.fill_batch([0, 1, 2], 2)
    after = paged_attention_decode(q, kp, vp, np.array(tables), np.array(lens))
    assert np.array_equal(after[[0, 2]], before[[0, 2]])
    K1 = np.concatenate([Kp, kn])
    V1 = np.concatenate([Vp, vn])
    for h in range(Hkv * G):
        ref = attention(to_f64(q[1, h]), to_f64(K1[:, h // G]), to_f64(V1[:, h // G]),
                        1 / math.sqrt(D))
        np.testing.assert_allclose(after[1, h], ref, rtol=0, atol=1e-13)
