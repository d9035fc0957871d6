"""Pins for the fp8 E4M3 codec of the quantized KV cache (CPU only).

Fixed by the format's definition (OCP 8-bit floating point, E4M3): code
points written out as numbers, every finite code decoding and re-encoding to
itself, encoding = the nearest finite value by brute-force search of the
whole table with ties to an even mantissa and saturation at 448, and
monotonicity."""
import math

import numpy as np
import pytest

from oracle import fp8


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x30, 0.5),
    (0x77, 240.0), (0x78, 256.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0)])
def test_code_points(code, value):
    assert fp8.e4m3_to_f64(code) == value
    assert fp8.f32_to_e4m3(value) == code


def test_special_codes():
    assert math.isnan(fp8.e4m3_to_f64(0x7F)) and math.isnan(fp8.e4m3_to_f64(0xFF))
    assert fp8.f32_to_e4m3(-0.0) == 0x80 and fp8.e4m3_to_f64(0x80) == 0.0
    assert fp8.f32_to_e4m3(float("nan")) == 0x7F
    for big in (448.0, 449.0, 463.9, 464.0, 1e6, float("inf")):
        assert fp8.f32_to_e4m3(big) == 0x7E and fp8.f32_to_e4m3(-big) == 0xFE


def test_every_finite_code_round_trips():
    for c in range(256):
        v = fp8.e4m3_to_f64(c)
        if not math.isnan(v):
            assert fp8.f32_to_e4m3(v) == c


def _nearest_by_search(y):
    """Brute force over the table: nearest finite value, ties to the even code."""
    finite = [(c, fp8.e4m3_to_f64(c)) for c in range(256)
              if not math.isnan(fp8.e4m3_to_f64(c))]
    if abs(y) >= 448.0:
        return 0x7E | (0x80 if y < 0 else 0)
    best = min(abs(v - y) for _, v in finite)
    cands = [c for c, v in finite if abs(v - y) == best]
    if len(cands) > 1:
        same_sign = [c for c in cands if (c & 0x80) == (0x80 if y < 0 or
                                                        math.copysign(1, y) < 0 else 0)]
        cands = same_sign or cands
        cands = [c for c in cands if (c & 1) == 0] or cands
    return cands[0]


def test_encoding_is_the_nearest_value():
    rng = np.random.default_rng(3)
    ys = np.concatenate([rng.normal(0, 4, 3000), rng.normal(0, 200, 500),
                         rng.uniform(-2 ** -6, 2 ** -6, 500)]).astype(np.float32)
    # exact midpoints between neighbouring codes: ties go to the even mantissa
    vals = sorted(v for v in fp8.DECODE if not math.isnan(v) and v >= 0)
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    for y in list(ys.astype(np.float64)) + mids + [-m for m in mids]:
        assert fp8.f32_to_e4m3(y) == _nearest_by_search(y), y


def test_monotone():
    xs = np.sort(np.random.default_rng(4).normal(0, 50, 4000))
    vals = [fp8.e4m3_to_f64(fp8.f32_to_e4m3(x)) for x in xs]
    assert all(a <= b for a, b in zip(vals, vals[1:]))


def test_per_head_scales():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, (6, 3, 8)).astype(np.float32)      # [tokens, heads, dims]
    scale = np.array([0.01, 0.5, 3.0], np.float32)
    codes = fp8.quantize(x, scale, head_axis=1)
    for h in range(3):
        want = [fp8.f32_to_e4m3(v) for v in (x[:, h] / scale[h]).reshape(-1).tolist()]
        assert codes[:, h].reshape(-1).tolist() == want
    back = fp8.dequantize(codes, scale, head_axis=1)
    # within half a step of the quantization grid (relative 1/16) or saturated
    rel = np.abs(back - x) / np.maximum(np.abs(x), 1e-30)
    sat = np.abs(x / scale[None, :, None]) >= 448
    assert np.all((rel <= 1 / 16 + 1e-7) | sat | (np.abs(x / scale[None, :, None]) < 2 ** -6))


def test_array_encoder_equals_the_definition():
    rng = np.random.default_rng(6)
    vals = sorted(v for v in fp8.DECODE if not math.isnan(v) and v >= 0)
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    ys = np.concatenate([rng.normal(0, 4, 20000), rng.normal(0, 300, 2000),
                         rng.uniform(-2 ** -5, 2 ** -5, 2000), mids, [-m for m in mids],
                         [0.0, -0.0, 448.0, -448.0, 1e9, -1e9, np.nan]]).astype(np.float32)
    got = fp8.encode(ys)
    want = [fp8.f32_to_e4m3(v) for v in ys.astype(np.float64).tolist()]
    assert got.tolist() == want


def test_fp8_cache_write_and_attention():
    """The cache write stores each token's quantized codes at its slot, and
    attention over an fp8 pool equals library attention over the dequantized
    contiguous K/V."""
    import torch
    from oracle.attention import paged_attention_decode
    from oracle.block_manager import BlockManager
    from oracle.cache_ops import reshape_and_cache
    from workloads import normal, pool_shapes
    rng = np.random.default_rng(8)
    Hkv, G, D, B = 2, 4, 32, 16
    lens = [1, 17, 40]
    N = sum(-(-L // B) for L in lens) + 2
    bm = BlockManager(N, B, rng.permutation(N))
    ks, vs = pool_shapes(N, Hkv, D, B, "fp8")
    k_pool = rng.integers(0, 0x7F, ks).astype(np.uint8)      # finite junk codes
    v_pool = rng.integers(0, 0x7F, vs).astype(np.uint8)
    k_scale = np.array([0.02, 0.05], np.float32)
    v_scale = np.array([0.03, 0.01], np.float32)
    Ks, Vs = [], []
    for s, L in enumerate(lens):
        bm.add_seq(s, 0)
        K, V = normal(rng, (L, Hkv, D), "bf16"), normal(rng, (L, Hkv, D), "bf16")
        slots = [bm.append_slot(s)[0] for _ in range(L)]
        k_pool, v_pool = reshape_and_cache(k_pool, v_pool, K, V, slots, k_scale, v_scale)
        kc = fp8.quantize((K.astype(np.uint32) << 16).view(np.float32), k_scale, 1)
        vc = fp8.quantize((V.astype(np.uint32) << 16).view(np.float32), v_scale, 1)
        for i, sl in enumerate(slots):
            b, o = divmod(sl, B)
            assert np.array_equal(k_pool[b, :, :, o, :].reshape(Hkv, D), kc[i])
            assert np.array_equal(v_pool[b, :, :, o], vc[i])
        Ks.append(fp8.dequantize(kc, k_scale, 1))
        Vs.append(fp8.dequantize(vc, v_scale, 1))
    tables, clens = bm.fill_batch(range(3), max(-(-L // B) for L in lens))
    q = normal(rng, (3, Hkv * G, D), "bf16")
    out = paged_attention_decode(q, k_pool, v_pool, np.array(tables), np.array(clens),
                                 k_scale=k_scale, v_scale=v_scale)
    from oracle.attention import to_f64
    for s, L in enumerate(lens):
        qs = torch.from_numpy(to_f64(q[s])).view(Hkv, G, 1, D)
        K = torch.from_numpy(Ks[s]).permute(1, 0, 2).reshape(Hkv, 1, L, D)
        V = torch.from_numpy(Vs[s]).permute(1, 0, 2).reshape(Hkv, 1, L, D)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qs, K.expand(Hkv, G, L, D), V.expand(Hkv, G, L, D), scale=1 / math.sqrt(D))
        np.testing.assert_allclose(out[s], ref.reshape(Hkv * G, D).numpy(), rtol=0, atol=1e-12)
