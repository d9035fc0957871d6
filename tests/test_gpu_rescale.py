"""GPU: score runs that move the softmax reference.

Both attention kernels keep, per query column, a reference maximum that may
trail the running maximum by up to 8 (base-2 exponent units) and move it only
when a score passes that margin; the weights gathered so far and their sum are
then scaled by 2^(old - new).  Unit-normal data almost never moves it after the
first tile, so here K is built so that every query head's scores follow a set
run along the context (the scaled score of token t is about c_t):

- rising: c_t = t / 4, so the reference moves every ~22 tokens (44 times in
  1,000), inside tiles, across tiles and in every partition of a split
  sequence;
- saw-tooth: runs of 200 tokens rising the same way, each starting 10 above
  the last, so the reference moves near the end of each run and earlier
  runs' weights shrink;
- falling: the first token scores highest and later weights underflow.

Outputs are compared with the fp64 oracle, which subtracts the exact maximum,
within the bounds of the other parity tests: decode (partitions merged in the
launch, with and without a plan; the matrix-core kernel for G >= 4 and the
VALU kernel below), multi-token queries, and bf16, fp32 and fp8 pools.

fp32 pools take the same runs at an eighth of the slope (scores up to about
30; the reference moves 6 times in 1,000 rising tokens).  At scores near 250
the fp32 rounding of the q.k sums alone moves the output by about 4e-5 of its
size (an fp64 simulation summing one product at a time, in random orders),
and the kernel's own sums moved it by 1.2e-5: past the 1e-5 relative bound
whatever the rest of the arithmetic does."""
import numpy as np
import pytest

import workloads as W
from oracle.attention import paged_attention_decode as ref_decode
from oracle.attention import paged_attention_prefill as ref_prefill
from oracle.block_manager import BlockManager
from oracle.cache_ops import reshape_and_cache as ref_cache
from tests.conftest import gpu_available
from tests.gpu_cases import NAN_BF16, check_attention, say, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

LENS = (1000, 777, 300, 64, 33, 1)
PATTERNS = ("rising", "sawtooth", "falling")


def bf16_bits(x) -> np.ndarray:
    """fp32 values rounded to bf16 (nearest, ties to even), as uint16 bits."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def target_scores(pattern: str, L: int, slope: float) -> np.ndarray:
    t = np.arange(L, dtype=np.float64)
    if pattern == "rising":
        return slope * t
    if pattern == "sawtooth":
        return slope * (t % 200) + 40.0 * slope * (t // 200)
    return 60.0 - slope * t


def build(rng, lens, Hkv, G, D, B, pattern, kv, queries_per_seq, rows=None):
    """Pools (NaN or NaN codes outside the sequences' tokens, placed through
    the reference block manager), tables, lengths and the query rows: each
    (sequence, KV head) has a direction u with u.u = D; its G query heads look
    along u, and token t's K is c_t u / sqrt(D) plus a little noise."""
    S = len(lens)
    N = sum(-(-L // B) for L in lens) + 5
    bm = BlockManager(N, B, rng.permutation(N))
    Ks, Vs, slots, qs = [], [], [], []
    for s, L in enumerate(lens):
        bm.add_seq(s, L)
        t = bm.tables[s]
        slots += [t[i // B] * B + i % B for i in range(L)]
        u = rng.standard_normal((Hkv, D))
        u *= np.sqrt(D) / np.linalg.norm(u, axis=1, keepdims=True)
        c = target_scores(pattern, L, 1 / 32 if kv == "f32" else 1 / 4)
        Ks.append(c[:, None, None] * u[None] / np.sqrt(D)
                  + 0.05 * rng.standard_normal((L, Hkv, D)))
        Vs.append(rng.standard_normal((L, Hkv, D)))
        nq = queries_per_seq[s]
        qs.append(np.repeat(u, G, axis=0)[None] + 0.05 * rng.standard_normal((nq, Hkv * G, D)))
    K, V = np.concatenate(Ks).astype(np.float32), np.concatenate(Vs).astype(np.float32)
    if rows is not None:  # the written K/V rows as the kernels take them, and their slots
        rows.update(k=K if kv == "f32" else bf16_bits(K), v=V if kv == "f32" else bf16_bits(V),
                    slots=np.asarray(slots, np.int64))
    q = np.concatenate(qs).astype(np.float32)
    q = q if kv == "f32" else bf16_bits(q)  # fp32 pools take fp32 queries, the others bf16
    slots = np.asarray(slots, np.int64)
    scales = {}
    if kv == "fp8":
        k_scale = (np.abs(K).max(axis=(0, 2)) / 400).astype(np.float32)
        v_scale = (np.abs(V).max(axis=(0, 2)) / 400).astype(np.float32)
        ks, vs = W.pool_shapes(N, Hkv, D, B, "fp8")
        kp, vp = np.full(ks, 0x7F, np.uint8), np.full(vs, 0x7F, np.uint8)
        kp, vp = ref_cache(kp, vp, bf16_bits(K), bf16_bits(V), slots, k_scale, v_scale)
        scales = {"k_scale": k_scale, "v_scale": v_scale}
    elif kv == "f32":
        ks, vs = W.pool_shapes(N, Hkv, D, B, "f32")
        kp, vp = np.full(ks, np.nan, np.float32), np.full(vs, np.nan, np.float32)
        kp, vp = ref_cache(kp, vp, K, V, slots)
    else:
        ks, vs = W.pool_shapes(N, Hkv, D, B, "bf16")
        kp, vp = np.full(ks, NAN_BF16, np.uint16), np.full(vs, NAN_BF16, np.uint16)
        kp, vp = ref_cache(kp, vp, bf16_bits(K), bf16_bits(V), slots)
    maxb = max(-(-L // B) for L in lens)
    tables, clens = bm.fill_batch(range(S), maxb)
    return kp, vp, np.asarray(tables, np.int32), np.asarray(clens, np.int32), q, scales


def _dev_scales(scales):
    import torch
    return {k: torch.from_numpy(v).cuda() for k, v in scales.items()}


def _pool(a):
    import torch
    return torch.from_numpy(a).cuda() if a.dtype == np.uint8 else to_dev(a)


# (kv, G, B, P, plan): matrix-core kernel (G >= 4) with partitions merged in the
# launch, planned and not; the VALU kernel (G = 1, 2); fp32 and fp8 pools
@pytest.mark.parametrize("kv,G,B,P,plan", [
    ("bf16", 4, 16, 256, True), ("bf16", 8, 32, 1024, False), ("bf16", 4, 16, 64, False),
    ("bf16", 1, 16, 128, True), ("f32", 2, 16, 256, False), ("fp8", 4, 16, 128, True)])
@pytest.mark.parametrize("pattern", PATTERNS)
def test_decode_follows_moving_reference(pkv, pattern, kv, G, B, P, plan):
    import torch
    say(f"case decode rescale {pattern} kv={kv} G={G} B={B} P={P} plan={plan}")
    rng = np.random.default_rng(4100 + 7 * G + B + P + PATTERNS.index(pattern))
    Hkv, D = 2, 128
    kp, vp, tables, clens, q, scales = build(rng, LENS, Hkv, G, D, B, pattern, kv,
                                             [1] * len(LENS))
    S = len(LENS)
    mcl = int(clens.max())
    out = torch.full((S, Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = pkv.attention_workspace(S, Hkv * G, D, mcl, P, device="cuda")
    pl = pkv.make_plan(clens, Hkv, B, tables.shape[1], mcl, P) if plan else None
    pkv.paged_attention_decode(out, to_dev(q), _pool(kp), _pool(vp),
                               torch.from_numpy(tables).cuda(), torch.from_numpy(clens).cuda(),
                               mcl, partition_size=P, workspace=ws, plan=pl,
                               **_dev_scales(scales))
    torch.cuda.synchronize()
    want = ref_decode(q, kp, vp, tables, clens, **scales)
    worst = check_attention(out.cpu().numpy(), want, "f32" if kv == "f32" else "bf16")
    say(f"  worst error {worst:.3e}")


@pytest.mark.parametrize("kv,G,B", [("bf16", 4, 16), ("bf16", 8, 32), ("bf16", 1, 16),
                                     ("fp8", 4, 16)])
@pytest.mark.parametrize("pattern", PATTERNS)
def test_prefill_follows_moving_reference(pkv, pattern, kv, G, B):
    import torch
    say(f"case prefill rescale {pattern} kv={kv} G={G} B={B}")
    rng = np.random.default_rng(4200 + 7 * G + B + PATTERNS.index(pattern))
    Hkv, D = 2, 128
    qlens = [70, 40, 300, 64, 10, 1]   # chunks at the ends, a whole prompt, a decode row
    kp, vp, tables, clens, q, scales = build(rng, LENS, Hkv, G, D, B, pattern, kv, qlens)
    starts = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    out = torch.full((q.shape[0], Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_attention_prefill(out, to_dev(q), _pool(kp), _pool(vp),
                                torch.from_numpy(tables).cuda(), torch.from_numpy(clens).cuda(),
                                torch.from_numpy(starts).cuda(), max(qlens),
                                **_dev_scales(scales))
    torch.cuda.synchronize()
    want = ref_prefill(q, kp, vp, tables, clens, qlens, **scales)
    worst = check_attention(out.cpu().numpy(), want, "bf16")
    say(f"  worst error {worst:.3e}")


@pytest.mark.parametrize("kv,G,P", [("bf16", 4, 256), ("bf16", 1, 128), ("fp8", 8, 128)])
@pytest.mark.parametrize("pattern", ("rising", "sawtooth"))
def test_decode_append_follows_moving_reference(pkv, pattern, kv, G, P):
    """The step's token, handed to the attention launch (new_key / new_value)
    and written by it, is the best-scoring token of a rising run: the launch
    takes it from the step's rows in its last tile, where the reference moves
    once more.  Output within the bound of the oracle over the pools with the
    token written; pools equal the oracle's bit for bit (codes for fp8)."""
    import torch
    from tests.gpu_cases import to_host_bits
    say(f"case decode append rescale {pattern} kv={kv} G={G} P={P}")
    rng = np.random.default_rng(4300 + 7 * G + P + (pattern == "sawtooth"))
    Hkv, D, B = 2, 128, 16
    rows = {}
    kp, vp, tables, clens, q, scales = build(rng, LENS, Hkv, G, D, B, pattern, kv,
                                             [1] * len(LENS), rows=rows)
    S = len(LENS)
    last = np.cumsum(LENS) - 1                 # each sequence's last row in the written rows
    new_k, new_v = rows["k"][last], rows["v"][last]
    kd, vd = kp.copy(), vp.copy()              # the pools before the step: last slots poisoned
    for sl in rows["slots"][last]:
        b, o = divmod(int(sl), B)
        kd[b, :, :, o, :] = 0x7F if kv == "fp8" else NAN_BF16
        vd[b, :, :, o] = 0x7F if kv == "fp8" else NAN_BF16
    mcl = int(clens.max())
    out = torch.full((S, Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
    kdev, vdev = _pool(kd), _pool(vd)
    ws = pkv.attention_workspace(S, Hkv * G, D, mcl, P, device="cuda")
    pl = pkv.make_plan(clens, Hkv, B, tables.shape[1], mcl, P)
    pkv.paged_attention_decode(out, to_dev(q), kdev, vdev, torch.from_numpy(tables).cuda(),
                               torch.from_numpy(clens).cuda(), mcl, partition_size=P,
                               workspace=ws, plan=pl, new_key=to_dev(new_k),
                               new_value=to_dev(new_v), **_dev_scales(scales))
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(kdev).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(to_host_bits(vdev).view(np.uint8), vp.view(np.uint8))
    want = ref_decode(q, kp, vp, tables, clens, **scales)
    worst = check_attention(out.cpu().numpy(), want, "bf16")
    say(f"  pools identical, worst error {worst:.3e}")
