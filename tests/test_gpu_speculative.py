"""Speculative decoding over the paged cache on the GPU, end to end through the
C ABI: each step every sequence takes slots for a few draft tokens through the
native block manager, their K/V are written by reshape_and_cache, the
multi-token kernel verifies them (each draft attends causally over the cache
and the drafts before it), a truncate gives back the rejected drafts, and the
next step's tokens overwrite the first rejected slots.  A final decode step
appends through the attention launch.  The whole pools are compared bit for
bit with the reference cache writes replayed on the host, and every attention
row with the fp64 reference within the bf16 bound; unused slots start as NaN."""
import numpy as np
import pytest

import workloads as W
from oracle.attention import paged_attention_decode as ref_decode
from oracle.attention import paged_attention_prefill as ref_prefill
from oracle.cache_ops import reshape_and_cache as ref_cache
from tests.conftest import gpu_available
from tests.gpu_cases import NAN_BF16, check_attention, say, to_dev, to_host_bits

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("B,G", [(16, 4), (32, 8), (16, 1)])
def test_speculative_steps(pkv, B, G):
    import torch
    say(f"case speculative B={B} G={G}")
    rng = np.random.default_rng(1900 + B + G)
    Hkv, D, S, N = 2, 128, 4, 64
    Hq = Hkv * G
    bm = pkv.BlockManager(N, B, rng.permutation(N).astype(np.int32))
    ks, vs = W.pool_shapes(N, Hkv, D, B, "bf16")
    hk, hv = np.full(ks, NAN_BF16, np.uint16), np.full(vs, NAN_BF16, np.uint16)
    dk, dv = to_dev(hk), to_dev(hv)

    def write(slots, K, V):
        nonlocal hk, hv
        slots = np.asarray(slots, np.int64)
        pkv.reshape_and_cache(to_dev(K), to_dev(V), dk, dv, torch.from_numpy(slots).cuda())
        hk, hv = ref_cache(hk, hv, K, V, slots)

    def batch():
        lens = [bm.seq_info(s)[0] for s in range(S)]
        maxb = max(1, max(-(-L // B) for L in lens))
        tables, clens = bm.fill_batch(range(S), maxb)
        return np.asarray(tables, np.int32), np.asarray(clens, np.int32)

    for s, L in enumerate((37, 64, 150, 5)):
        bm.add_seq(s, L)
        write(bm.slots(s, 0, L)[:L], W.normal(rng, (L, Hkv, D), "bf16"),
              W.normal(rng, (L, Hkv, D), "bf16"))
    rejected = 0
    for step in range(4):
        k = [int(x) for x in rng.integers(1, 5, S)]
        slots = []
        for s in range(S):
            for _ in range(k[s]):
                slot, src, dst = bm.append_slot(s)
                assert src < 0          # no sharing here: no copy-on-write
                slots.append(slot)
        T = sum(k)
        write(slots, W.normal(rng, (T, Hkv, D), "bf16"), W.normal(rng, (T, Hkv, D), "bf16"))
        tables, clens = batch()
        q = W.normal(rng, (T, Hq, D), "bf16")
        out = torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        starts = np.concatenate([[0], np.cumsum(k)]).astype(np.int32)
        pkv.paged_attention_prefill(out, to_dev(q), dk, dv, torch.from_numpy(tables).cuda(),
                                    torch.from_numpy(clens).cuda(),
                                    torch.from_numpy(starts).cuda(), max(k))
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(dk).view(np.uint8), hk.view(np.uint8))
        assert np.array_equal(to_host_bits(dv).view(np.uint8), hv.view(np.uint8))
        worst = check_attention(out.cpu().numpy(), ref_prefill(q, hk, hv, tables, clens, k),
                                "bf16")
        # the verifier keeps j of the k drafts of each sequence
        for s in range(S):
            j = int(rng.integers(0, k[s] + 1))
            rejected += k[s] - j
            bm.truncate(s, int(clens[s]) - k[s] + j)
        say(f"  step {step}: drafts {k}, worst error {worst:.3e}")
    assert rejected > 0
    # a plain decode step after the last verification: one token per sequence,
    # written by the attention launch over the first rejected slot
    slots, pairs = bm.append_slots(list(range(S)))
    assert len(pairs) == 0
    kn, vn = W.normal(rng, (S, Hkv, D), "bf16"), W.normal(rng, (S, Hkv, D), "bf16")
    tables, clens = batch()
    q = W.normal(rng, (S, Hq, D), "bf16")
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    mcl = int(clens.max())
    ws = pkv.attention_workspace(S, Hq, D, mcl, 64, device="cuda")
    pkv.paged_attention_decode(out, to_dev(q), dk, dv, torch.from_numpy(tables).cuda(),
                               torch.from_numpy(clens).cuda(), mcl, partition_size=64,
                               workspace=ws, new_key=to_dev(kn), new_value=to_dev(vn))
    torch.cuda.synchronize()
    hk, hv = ref_cache(hk, hv, kn, vn, np.asarray(slots, np.int64))
    assert np.array_equal(to_host_bits(dk).view(np.uint8), hk.view(np.uint8))
    assert np.array_equal(to_host_bits(dv).view(np.uint8), hv.view(np.uint8))
    check_attention(out.cpu().numpy(), ref_decode(q, hk, hv, tables, clens), "bf16")
