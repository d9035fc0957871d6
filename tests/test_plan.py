"""Host work plan (pkv_attention_plan): exactly the batch's non-empty
(sequence, KV head, partition) items, each once, largest first, then the rows
the reduce must merge (CPU only; the plan is a schedule, so it is checked
against the partition rule it encodes rather than against the oracle)."""
import numpy as np
import pytest


def expected_items(lens, Hkv, B, max_blocks, mcl, P):
    cap = max_blocks * B
    nparts = max(1, -(-min(mcl, cap) // P))
    items, merge = {}, []
    for s, L0 in enumerate(lens):
        L = min(int(L0), cap)
        n = 0 if L <= 0 else min(-(-L // P), nparts)
        for p in range(max(n, 1)):
            size = 0 if L <= 0 else min(P, L - p * P)
            for g in range(Hkv):
                items[(s, g, p)] = (int(L0), size)   # the length as given
        if n > 1:
            merge += [s * Hkv + g for g in range(Hkv)]
    return items, merge


@pytest.mark.parametrize("seed", range(12))
def test_plan_lists_each_item_once_largest_first(pkv, seed):
    rng = np.random.default_rng(900 + seed)
    B = int(rng.choice([16, 32]))
    P = int(rng.choice([32, 64, 256, 512])) // B * B or B
    P = max(P, 32)
    if P % B:
        P = B * 2
    Hkv = int(rng.integers(1, 9))
    S = int(rng.integers(0, 40))
    max_blocks = int(rng.integers(1, 80))
    lens = rng.integers(-2, max_blocks * B + 40, size=S).astype(np.int32)
    lens[rng.random(S) < 0.15] = 0
    mcl = int(max(lens.max(initial=0), 0))
    words, n_items, n_merge = pkv.attention_plan(lens, Hkv, B, max_blocks, mcl, P)
    assert words.shape[0] == 4 * n_items + n_merge
    assert words.shape[0] <= pkv.attention_plan_words(S, Hkv, B, max_blocks, mcl, P) or S == 0
    items, merge = expected_items(lens, Hkv, B, max_blocks, mcl, P)
    recs = words[:4 * n_items].reshape(-1, 4)
    got = {}
    for s, g, p, L in recs.tolist():
        assert (s, g, p) not in got
        got[(s, g, p)] = L
    assert set(got) == set(items)
    sizes = [items[(s, g, p)][1] for s, g, p, _ in recs.tolist()]
    assert all(a >= b for a, b in zip(sizes, sizes[1:]))
    for key, L in got.items():
        assert L == items[key][0]
    assert words[4 * n_items:].tolist() == merge


def test_plan_capacity_and_validation(pkv):
    lens = np.array([600, 0, 1500], np.int32)
    cap = pkv.attention_plan_words(3, 8, 16, 100, 1500, 512)
    assert cap == 3 * 8 * (4 * 3 + 1)
    words, n_items, n_merge = pkv.attention_plan(lens, 8, 16, 100, 1500, 512)
    assert (n_items, n_merge) == (8 * (2 + 1 + 3), 8 * 2)
    # the first records are full 512-token partitions, the zero-length sequence's
    # empty item comes last
    recs = words[:4 * n_items].reshape(-1, 4)
    assert recs[0][3] >= 512 and recs[-1].tolist()[3] == 0
    # too small a buffer: counts are reported, nothing is written, EINVAL
    import ctypes
    buf = np.full(10, -7, np.int32)
    ni, nm = ctypes.c_int32(), ctypes.c_int32()
    st = pkv.lib.pkv_attention_plan(lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 3, 8, 16,
                                    100, 1500, 512,
                                    buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 10,
                                    ctypes.byref(ni), ctypes.byref(nm))
    assert st == pkv.PKV_EINVAL and (ni.value, nm.value) == (n_items, n_merge)
    assert (buf == -7).all()
    # partition rules are those of the attention call
    with pytest.raises(pkv.PkvError):
        pkv.attention_plan(lens, 8, 16, 100, 1500, 48)
    with pytest.raises(pkv.PkvError):
        pkv.attention_plan(lens, 8, 16, 100, 1500, 4096)
    # an empty batch plans nothing
    words, n_items, n_merge = pkv.attention_plan(np.zeros(0, np.int32), 8, 16, 100, 0, 512)
    assert (words.size, n_items, n_merge) == (0, 0, 0)
