"""GPU parity of swap_blocks: block copies between the device pool and a pinned
host pool, both directions, compared bit for bit with the same copies done on
the host arrays (whole pools; the host pool starts NaN-poisoned, so a write to
the wrong block or a skipped pair that is not skipped shows up)."""
import numpy as np
import pytest

import workloads as W
from tests.conftest import gpu_available
from tests.gpu_cases import NAN_BF16, say, to_dev, to_host_bits

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _pinned_copy(a):
    import torch
    t = to_dev(a).cpu().pin_memory()
    assert t.is_pinned()
    return t


@pytest.mark.parametrize("dtype,Hkv,D,B", [("bf16", 8, 128, 16), ("bf16", 2, 64, 32),
                                           ("f32", 4, 128, 16)])
def test_swap_blocks_round_trip(pkv, dtype, Hkv, D, B):
    import torch
    say(f"case swap_blocks {dtype} Hkv={Hkv} D={D} B={B}")
    rng = np.random.default_rng(42 + Hkv + D + B)
    N, NH = 40, 24
    ks, vs = W.pool_shapes(N, Hkv, D, B, dtype)
    hks, hvs = W.pool_shapes(NH, Hkv, D, B, dtype)
    dk, dv = W.normal(rng, ks, dtype), W.normal(rng, vs, dtype)
    nan = NAN_BF16 if dtype == "bf16" else np.float32(np.nan)
    hk = np.full(hks, nan, dk.dtype)
    hv = np.full(hvs, nan, dv.dtype)

    k_dev, v_dev = to_dev(dk), to_dev(dv)
    k_host, v_host = _pinned_copy(hk), _pinned_copy(hv)

    # swap-out: 10 device blocks to host blocks, plus pairs that must be skipped
    src = rng.choice(N, 10, replace=False)
    dst = rng.choice(NH, 10, replace=False)
    out_pairs = np.stack([src, dst], 1).astype(np.int32)
    skipped = np.array([[N, 0], [0, NH], [-1, 1]], np.int32)
    pairs = np.concatenate([out_pairs, skipped])
    pkv.swap_blocks(k_host, v_host, k_dev, v_dev, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    for s_, d_ in out_pairs:
        hk[d_] = dk[s_]
        hv[d_] = dv[s_]
    assert np.array_equal(to_host_bits(k_host).view(np.uint8), hk.view(np.uint8))
    assert np.array_equal(to_host_bits(v_host).view(np.uint8), hv.view(np.uint8))

    # swap-in: those host blocks back into other device blocks
    back = rng.choice(np.setdiff1d(np.arange(N), src), 10, replace=False)
    in_pairs = np.stack([dst, back], 1).astype(np.int32)
    pkv.swap_blocks(k_dev, v_dev, k_host, v_host, torch.from_numpy(in_pairs).cuda())
    torch.cuda.synchronize()
    for s_, d_ in in_pairs:
        dk[d_] = hk[s_]
        dv[d_] = hv[s_]
    assert np.array_equal(to_host_bits(k_dev).view(np.uint8), dk.view(np.uint8))
    assert np.array_equal(to_host_bits(v_dev).view(np.uint8), dv.view(np.uint8))


def test_swap_blocks_rejects_pageable_host_memory_in_the_binding(pkv):
    import torch
    ks, vs = W.pool_shapes(4, 2, 64, 16, "bf16")
    k_dev = torch.zeros(ks, dtype=torch.bfloat16, device="cuda")
    v_dev = torch.zeros(vs, dtype=torch.bfloat16, device="cuda")
    k_page = torch.zeros(ks, dtype=torch.bfloat16)
    v_page = torch.zeros(vs, dtype=torch.bfloat16)
    pairs = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        pkv.swap_blocks(k_page, v_page, k_dev, v_dev, pairs)
