"""GPU parity of the fp8 E4M3 KV cache against the reference, through the C ABI.

Cache writes: the codes the kernel stores equal the reference encoder's bit
for bit (saturation, the subnormal range, exact ties, signed zero and NaN
included).  Attention over fp8 pools: within the bf16 bound (2e-3 max abs) of
the fp64 reference over the dequantized values, planned and unplanned, with
NaN codes in every slot that holds no token.  Block copies move fp8 blocks
bit for bit."""
import numpy as np
import pytest

import workloads as W
from oracle import fp8
from oracle.attention import paged_attention_decode as ref_decode
from oracle.block_manager import BlockManager
from oracle.cache_ops import reshape_and_cache as ref_cache
from tests.conftest import gpu_available
from tests.gpu_cases import Bookkeeping, check_attention, say, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

NAN8 = np.uint8(0x7F)


def _u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _bits_of(x32):
    """fp32 values that are exact in bf16 -> bf16 bit patterns."""
    return (np.asarray(x32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_fp8_cache_write_bit_exact(pkv):
    import torch
    say("case fp8 reshape_and_cache")
    rng = np.random.default_rng(61)
    Hkv, D, B, N, T = 4, 128, 16, 24, 40
    k_scale = np.array([1.0, 0.125, 0.0123, 3.7], np.float32)
    v_scale = np.array([0.5, 1.0, 0.02, 0.003], np.float32)
    K = W.normal(rng, (T, Hkv, D), "bf16")
    V = W.normal(rng, (T, Hkv, D), "bf16")
    # edge values in the first rows: exact midpoints between codes (ties, exact
    # at power-of-two scales), saturation, the subnormal range, +-0, NaN
    vals = sorted(v for v in fp8.DECODE if not np.isnan(v) and v >= 0)
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    edge = np.array(mids + [-m for m in mids] + [500.0, -16384.0, 2 ** -12, 3 * 2 ** -10, 0.0,
                                                 -0.0], np.float32)
    edge_bits = _bits_of(edge)
    assert np.array_equal(((edge_bits.astype(np.uint32) << 16).view(np.float32)), edge)
    flat = K[:8, :2].reshape(-1)
    flat[:edge_bits.size] = edge_bits
    K[:8, :2] = flat.reshape(8, 2, D)
    V[0, 0, :4] = np.array([0x7FC1, 0xFFC1, 0x0000, 0x8000], np.uint16)   # NaN, -NaN, 0, -0
    slots = rng.permutation(N * B)[:T].astype(np.int64)
    slots[3] = -1                                                       # skipped
    ks, vs = W.pool_shapes(N, Hkv, D, B, "fp8")
    kp0 = rng.integers(0, 0x7F, ks).astype(np.uint8)
    vp0 = rng.integers(0, 0x7F, vs).astype(np.uint8)
    kp, vp = _u8(kp0), _u8(vp0)
    pkv.reshape_and_cache(to_dev(K), to_dev(V), kp, vp, torch.from_numpy(slots).cuda(),
                          k_scale=torch.from_numpy(k_scale).cuda(),
                          v_scale=torch.from_numpy(v_scale).cuda())
    torch.cuda.synchronize()
    rk, rv = ref_cache(kp0, vp0, K, V, slots, k_scale, v_scale)
    assert np.array_equal(kp.cpu().numpy(), rk)
    assert np.array_equal(vp.cpu().numpy(), rv)


def _fp8_pools(rng, lens, Hkv, D, B, k_scale, v_scale, extra=4):
    """fp8 pools holding each sequence's quantized K/V through the reference
    block manager (shuffled free queue); every other slot holds the NaN code."""
    need = sum(-(-L // B) for L in lens)
    N = need + extra
    bm = BlockManager(N, B, rng.permutation(N))
    ks, vs = W.pool_shapes(N, Hkv, D, B, "fp8")
    kp, vp = np.full(ks, NAN8, np.uint8), np.full(vs, NAN8, np.uint8)
    slots, Ks, Vs = [], [], []
    for s, L in enumerate(lens):
        bm.add_seq(s, L)
        t = bm.tables[s]
        slots += [t[i // B] * B + i % B for i in range(L)]
        Ks.append(W.normal(rng, (L, Hkv, D), "bf16"))
        Vs.append(W.normal(rng, (L, Hkv, D), "bf16"))
    kp, vp = ref_cache(kp, vp, np.concatenate(Ks), np.concatenate(Vs), np.asarray(slots),
                       k_scale, v_scale)
    maxb = max(-(-L // B) for L in lens)
    tables, clens = bm.fill_batch(range(len(lens)), maxb)
    return kp, vp, np.asarray(tables, np.int32), np.asarray(clens, np.int32), N


LENS = (1, 2, 15, 16, 17, 33, 100, 511, 512, 513, 1030, 1300)


# partitions of 96 tokens end inside a 64-token fp8 tile; shared: cached loads
@pytest.mark.parametrize("G,D,B,P,plan,shared", [
    (4, 128, 16, 512, True, False), (8, 128, 16, 256, False, False),
    (8, 128, 32, 512, True, False), (4, 64, 32, 128, False, False),
    (8, 64, 16, 1024, True, False), (4, 128, 32, 96, False, False),
    (8, 128, 16, 96, True, True), (4, 128, 16, 512, False, True),
    (1, 128, 16, 512, True, False), (2, 128, 32, 256, False, False),
    (1, 64, 32, 96, False, True), (2, 64, 16, 1024, True, False),
    (4, 128, 16, 2048, True, False), (8, 128, 32, 4096, False, False)])
def test_fp8_attention_matches_reference(pkv, G, D, B, P, plan, shared):
    import torch
    say(f"case fp8 attention G={G} D={D} B={B} P={P} plan={plan} shared={shared}")
    rng = np.random.default_rng(70 + G + D + B + P)
    Hkv = 2
    k_scale = rng.uniform(0.004, 0.03, Hkv).astype(np.float32)
    v_scale = rng.uniform(0.004, 0.03, Hkv).astype(np.float32)
    kp, vp, tables, clens, N = _fp8_pools(rng, LENS, Hkv, D, B, k_scale, v_scale)
    S = len(LENS)
    q = W.normal(rng, (S, Hkv * G, D), "bf16")
    mcl = int(clens.max())
    out = torch.full((S, Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = pkv.attention_workspace(S, Hkv * G, D, mcl, P, device="cuda")
    pl = pkv.make_plan(clens, Hkv, B, tables.shape[1], mcl, P) if plan else None
    pkv.paged_attention_decode(out, to_dev(q), _u8(kp), _u8(vp), torch.from_numpy(tables).cuda(),
                               torch.from_numpy(clens).cuda(), mcl, partition_size=P,
                               workspace=ws, plan=pl, shared_kv=shared,
                               k_scale=torch.from_numpy(k_scale).cuda(),
                               v_scale=torch.from_numpy(v_scale).cuda())
    torch.cuda.synchronize()
    want = ref_decode(q, kp, vp, tables, clens, k_scale=k_scale, v_scale=v_scale)
    worst = check_attention(out.cpu().numpy(), want, "bf16")
    say(f"  worst error {worst:.3e}")


def test_fp8_block_copies_bit_exact(pkv):
    import torch
    say("case fp8 copy_blocks")
    rng = np.random.default_rng(75)
    ks, vs = W.pool_shapes(12, 2, 128, 16, "fp8")
    kp0 = rng.integers(0, 256, ks).astype(np.uint8)
    vp0 = rng.integers(0, 256, vs).astype(np.uint8)
    kp, vp = _u8(kp0), _u8(vp0)
    pairs = np.array([[0, 5], [3, 7], [11, 2]], np.int32)
    pkv.copy_blocks(kp, vp, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    for s_, d_ in pairs:
        kp0[d_], vp0[d_] = kp0[s_], vp0[s_]
    assert np.array_equal(kp.cpu().numpy(), kp0) and np.array_equal(vp.cpu().numpy(), vp0)


@pytest.mark.parametrize("G,D,B,P,plan", [(4, 128, 16, 512, True), (8, 128, 32, 256, False),
                                          (4, 64, 16, 96, True), (8, 64, 32, 1024, False),
                                          (1, 128, 16, 512, True), (2, 64, 32, 96, False)])
def test_fp8_append_in_the_attention_launch(pkv, G, D, B, P, plan):
    """new_key / new_value (bf16) are encoded, written into each sequence's last
    slot and attended to in the same launch: pools bit-identical to the cache
    write, output within the bf16 bound of the reference over those pools."""
    import torch
    say(f"case fp8 append G={G} D={D} B={B} P={P} plan={plan}")
    rng = np.random.default_rng(90 + G + D + B + P)
    Hkv = 2
    lens = (1, 2, 16, 17, 32, 33, 63, 64, 65, 96, 97, 511, 512, 513, 1025)
    k_scale = rng.uniform(0.004, 0.03, Hkv).astype(np.float32)
    v_scale = rng.uniform(0.004, 0.03, Hkv).astype(np.float32)
    N = sum(-(-L // B) for L in lens) + 3
    bm = BlockManager(N, B, rng.permutation(N))
    ks, vs = W.pool_shapes(N, Hkv, D, B, "fp8")
    kp, vp = np.full(ks, NAN8, np.uint8), np.full(vs, NAN8, np.uint8)
    slots, Ks, Vs, new_slots = [], [], [], []
    for s, L in enumerate(lens):
        bm.add_seq(s, L - 1)
        t = bm.tables[s]
        slots += [t[i // B] * B + i % B for i in range(L - 1)]
        Ks.append(W.normal(rng, (L - 1, Hkv, D), "bf16"))
        Vs.append(W.normal(rng, (L - 1, Hkv, D), "bf16"))
        new_slots.append(bm.append_slot(s)[0])
    kp, vp = ref_cache(kp, vp, np.concatenate(Ks), np.concatenate(Vs), np.asarray(slots),
                       k_scale, v_scale)
    S = len(lens)
    tables, clens = bm.fill_batch(range(S), max(-(-L // B) for L in lens))
    tables, clens = np.asarray(tables, np.int32), np.asarray(clens, np.int32)
    assert clens.tolist() == list(lens)
    k_new = W.normal(rng, (S, Hkv, D), "bf16")
    v_new = W.normal(rng, (S, Hkv, D), "bf16")
    q = W.normal(rng, (S, Hkv * G, D), "bf16")
    mcl = int(clens.max())
    dk, dv = _u8(kp), _u8(vp)
    out = torch.full((S, Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = pkv.attention_workspace(S, Hkv * G, D, mcl, P, device="cuda")
    pl = pkv.make_plan(clens, Hkv, B, tables.shape[1], mcl, P) if plan else None
    pkv.paged_attention_decode(out, to_dev(q), dk, dv, torch.from_numpy(tables).cuda(),
                               torch.from_numpy(clens).cuda(), mcl, partition_size=P,
                               workspace=ws, plan=pl, new_key=to_dev(k_new),
                               new_value=to_dev(v_new),
                               k_scale=torch.from_numpy(k_scale).cuda(),
                               v_scale=torch.from_numpy(v_scale).cuda())
    torch.cuda.synchronize()
    rk, rv = ref_cache(kp, vp, k_new, v_new, np.asarray(new_slots), k_scale, v_scale)
    assert np.array_equal(dk.cpu().numpy(), rk)
    assert np.array_equal(dv.cpu().numpy(), rv)
    want = ref_decode(q, rk, rv, tables, clens, k_scale=k_scale, v_scale=v_scale)
    worst = check_attention(out.cpu().numpy(), want, "bf16")
    say(f"  worst error {worst:.3e}")


@pytest.mark.parametrize("G", [1, 4])
def test_fp8_subnormal_codes_decode_exactly(pkv, G):
    """A KV head whose scale is large stores mostly subnormal codes (exponent
    field 0): the widening must keep them (no flush to zero) in both kernels."""
    import torch
    say(f"case fp8 subnormal codes G={G}")
    rng = np.random.default_rng(130 + G)
    Hkv, D, B, P = 2, 128, 16, 512
    k_scale = np.array([0.02, 60.0], np.float32)
    v_scale = np.array([0.02, 60.0], np.float32)
    lens = (5, 40, 700)
    kp, vp, tables, clens, N = _fp8_pools(rng, lens, Hkv, D, B, k_scale, v_scale)
    used = np.zeros(N, bool)
    for s, L in enumerate(lens):
        used[tables[s, :-(-L // B)]] = True
    codes = kp[used][:, 1]
    sub = ((codes & 0x78) == 0) & ((codes & 7) != 0)
    assert sub.mean() > 0.3, sub.mean()        # head 1 is mostly subnormal codes
    S = len(lens)
    q = W.normal(rng, (S, Hkv * G, D), "bf16")
    mcl = int(clens.max())
    out = torch.full((S, Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = pkv.attention_workspace(S, Hkv * G, D, mcl, P, device="cuda")
    pkv.paged_attention_decode(out, to_dev(q), _u8(kp), _u8(vp), torch.from_numpy(tables).cuda(),
                               torch.from_numpy(clens).cuda(), mcl, partition_size=P,
                               workspace=ws, k_scale=torch.from_numpy(k_scale).cuda(),
                               v_scale=torch.from_numpy(v_scale).cuda())
    torch.cuda.synchronize()
    want = ref_decode(q, kp, vp, tables, clens, k_scale=k_scale, v_scale=v_scale)
    worst = check_attention(out.cpu().numpy(), want, "bf16")
    say(f"  worst error {worst:.3e}")


@pytest.mark.parametrize("name", ["llama8b_gqa", "long70b_b16"])
def test_fp8_full_config(pkv, name):
    """Full-size workloads over fp8 pools in the benchmark's launch configuration
    (host plan; the step's tokens encoded and written by the attention launch):
    the oracle's block manager reproduces the product's tables and slots; whole
    pools bit-exact against the reference fp8 cache write; every (sequence,
    query head) row within the bf16 bound of the fp64 reference over the
    dequantized pools.  Pools hold random finite codes, NaN codes in every slot
    that holds no token."""
    import torch
    from oracle.attention import valid_slot_mask
    say(f"case fp8 {name} (full size)")
    w = W.make(name, pools=False)
    c = w.cfg
    bk = Bookkeeping(pkv, w)
    ids = list(range(c.S))
    max_blocks = bk.max_blocks
    assert len(bk.pairs) == 0
    pre_tables, pre_lens = bk.ref_pre_tables, bk.ref_pre_lens
    tables, lens = bk.tables, bk.lens
    rng = np.random.default_rng(2000 + c.seed)
    ks, vs = W.pool_shapes(w.num_blocks, c.Hkv, c.D, c.B, "fp8")

    def codes(shape):   # finite E4M3 codes below 4 in magnitude, random sign
        return (rng.integers(0, 0x50, shape, dtype=np.uint8)
                | (rng.integers(0, 2, shape, dtype=np.uint8) << 7))

    kp, vp = codes(ks), codes(vs)
    bi, oi = np.nonzero(~valid_slot_mask(pre_tables, pre_lens, w.num_blocks, c.B))
    kp[bi, :, :, oi, :] = NAN8
    vp[bi, :, :, oi] = NAN8
    k_scale = np.linspace(0.02, 0.03, c.Hkv).astype(np.float32)
    v_scale = np.linspace(0.03, 0.02, c.Hkv).astype(np.float32)
    append = len(w.step_ids) > 0
    assert not append or list(w.step_ids) == ids
    mcl = int(lens.max())
    P = c.partition_size
    dk, dv = _u8(kp), _u8(vp)
    out = torch.full((c.S, c.Hq, c.D), float("nan"), dtype=torch.float32, device="cuda")
    ws = pkv.attention_workspace(c.S, c.Hq, c.D, mcl, P, device="cuda")
    pl = pkv.make_plan(lens, c.Hkv, c.B, max_blocks, mcl, P)
    pkv.paged_attention_decode(out, to_dev(w.q), dk, dv, torch.from_numpy(tables).cuda(),
                               torch.from_numpy(lens).cuda(), mcl, partition_size=P,
                               workspace=ws, plan=pl,
                               new_key=to_dev(w.k_new) if append else None,
                               new_value=to_dev(w.v_new) if append else None,
                               k_scale=torch.from_numpy(k_scale).cuda(),
                               v_scale=torch.from_numpy(v_scale).cuda())
    torch.cuda.synchronize()
    say("  device done")
    if append:
        kp, vp = ref_cache(kp, vp, w.k_new, w.v_new, bk.ref_slots, k_scale, v_scale)
    assert np.array_equal(dk.cpu().numpy(), kp)
    assert np.array_equal(dv.cpu().numpy(), vp)
    want = ref_decode(w.q, kp, vp, bk.ref_tables, bk.ref_lens, k_scale=k_scale, v_scale=v_scale)
    worst = check_attention(out.cpu().numpy(), want, "bf16")
    say(f"  all {c.S * c.Hq} rows, worst error {worst:.3e}")
