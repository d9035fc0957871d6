"""GPU parity of the multi-token (chunked prefill / prefix-hit) attention kernel
against the fp64 reference, through the C ABI.

Pools are filled through the reference block manager with a shuffled free
queue, and every slot that holds no token is NaN, so a read past a sequence's
end or into a foreign block shows up.  Bound: bf16 max abs error 2e-3, as for
decode.  Also the bit-exact identity chunked == one pass, and one query agrees
with the decode kernel."""
import numpy as np
import pytest

import workloads as W
from oracle.attention import paged_attention_prefill as ref_prefill
from oracle.block_manager import BlockManager
from tests.conftest import gpu_available
from tests.gpu_cases import NAN_BF16, check_attention, say, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def build(rng, lens, Hkv, D, B, extra=5):
    """A NaN pool holding random K/V for each sequence's tokens, placed through
    the reference block manager; returns pools, tables [S, maxb] and lens."""
    need = sum(-(-L // B) for L in lens)
    N = need + extra
    bm = BlockManager(N, B, rng.permutation(N))
    ks, vs = W.pool_shapes(N, Hkv, D, B, "bf16")
    kp, vp = np.full(ks, NAN_BF16, np.uint16), np.full(vs, NAN_BF16, np.uint16)
    for s, L in enumerate(lens):
        bm.add_seq(s, L)
        t = bm.tables[s]
        K = W.normal(rng, (L, Hkv, D), "bf16")
        V = W.normal(rng, (L, Hkv, D), "bf16")
        for i in range(L):
            b, o = t[i // B], i % B
            kp[b, :, :, o, :] = K[i].reshape(Hkv, D // 8, 8)
            vp[b, :, :, o] = V[i]
    maxb = max(1, max(-(-L // B) for L in lens))
    tables, clens = bm.fill_batch(range(len(lens)), maxb)
    return kp, vp, np.asarray(tables, np.int32), np.asarray(clens, np.int32)


def run(pkv, q, kp, vp, tables, clens, qlens, starts=None):
    import torch
    if starts is None:
        starts = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = q.shape[0]
    out = torch.full((T, q.shape[1], q.shape[2]), float("nan"), dtype=torch.float32,
                     device="cuda")
    pkv.paged_attention_prefill(out, to_dev(q), to_dev(kp), to_dev(vp),
                                torch.from_numpy(tables).cuda(), torch.from_numpy(clens).cuda(),
                                torch.from_numpy(np.asarray(starts, np.int32)).cuda(),
                                int(max(qlens) if len(qlens) else 0))
    torch.cuda.synchronize()
    return out.cpu().numpy()


LENS = (1, 17, 100, 1300, 513, 40, 64)
QLENS = (1, 17, 37, 5, 70, 0, 64)       # decode, whole prompts, chunks, a prefix hit, empty


@pytest.mark.parametrize("G,D,B", [(1, 128, 16), (2, 64, 32), (4, 128, 16), (4, 128, 32),
                                   (8, 128, 16), (8, 64, 16), (1, 64, 32), (2, 128, 16)])
def test_prefill_matches_reference(pkv, G, D, B):
    say(f"case prefill G={G} D={D} B={B}")
    rng = np.random.default_rng(900 + G * 7 + D + B)
    Hkv = 2
    kp, vp, tables, clens = build(rng, LENS, Hkv, D, B)
    q = W.normal(rng, (sum(QLENS), Hkv * G, D), "bf16")
    got = run(pkv, q, kp, vp, tables, clens, QLENS)
    want = ref_prefill(q, kp, vp, tables, clens, QLENS)
    worst = check_attention(got, want, "bf16")
    say(f"  worst error {worst:.3e}")


def test_chunked_equals_one_pass_bit_exact(pkv):
    """Rows of a 300-token prompt attended as chunks of 100 + 120 + 80 over the
    growing cache equal the rows of one 300-token pass, bit for bit."""
    say("case prefill chunking identity")
    rng = np.random.default_rng(77)
    Hkv, G, D, B = 8, 4, 128, 16
    L = 300
    kp, vp, tables, clens = build(rng, [L], Hkv, D, B)
    q = W.normal(rng, (L, Hkv * G, D), "bf16")
    whole = run(pkv, q, kp, vp, tables, clens, [L])
    done = 0
    for chunk in (100, 120, 80):
        part = run(pkv, q[done:done + chunk], kp, vp, tables,
                   np.array([done + chunk], np.int32), [chunk])
        assert np.array_equal(part.view(np.uint32), whole[done:done + chunk].view(np.uint32))
        done += chunk


@pytest.mark.parametrize("G,B", [(4, 16), (8, 32)])
def test_one_query_matches_decode(pkv, G, B):
    """One query per sequence: the multi-token kernel's rows agree with the
    decode kernel's and with the fp64 reference.  The two kernels order the
    weights' sums differently (the multi-token one keeps a trailing reference
    maximum and a different token order inside an MFMA), so they agree to
    rounding, not bit for bit."""
    import torch
    say(f"case prefill vs decode G={G} B={B}")
    rng = np.random.default_rng(81 + G + B)
    Hkv, D = 2, 128
    lens = (1, 15, 16, 33, 500, 1000)
    kp, vp, tables, clens = build(rng, lens, Hkv, D, B)
    q = W.normal(rng, (len(lens), Hkv * G, D), "bf16")
    got = run(pkv, q, kp, vp, tables, clens, [1] * len(lens))
    out = torch.empty((len(lens), Hkv * G, D), dtype=torch.float32, device="cuda")
    pkv.paged_attention_decode(out, to_dev(q), to_dev(kp), to_dev(vp),
                               torch.from_numpy(tables).cuda(), torch.from_numpy(clens).cuda(),
                               int(max(lens)), partition_size=1024)
    torch.cuda.synchronize()
    dec = out.cpu().numpy()
    want = ref_prefill(q, kp, vp, tables, clens, [1] * len(lens))
    check_attention(got, want, "bf16")
    check_attention(dec, want, "bf16")
    diff = float(np.abs(got.astype(np.float64) - dec).max())
    say(f"  prefill vs decode max difference {diff:.3e}")
    assert diff <= 1e-4


def test_rows_outside_the_batch_are_not_written(pkv):
    """A sequence with more rows than tokens gets its last L rows; one whose rows
    run past T gets none; the others are unaffected."""
    say("case prefill malformed offsets")
    rng = np.random.default_rng(91)
    Hkv, G, D, B = 2, 4, 64, 16
    lens = (5, 30, 20)
    kp, vp, tables, clens = build(rng, lens, Hkv, D, B)
    starts = np.array([0, 8, 18, 40], np.int32)      # 8 rows for 5 tokens; 10; 22 > T
    T = 30
    q = W.normal(rng, (T, Hkv * G, D), "bf16")
    got = run(pkv, q, kp, vp, tables, clens, [8, 10, 22], starts=starts)
    assert np.isnan(got[0:3]).all() and np.isnan(got[18:]).all()
    want0 = ref_prefill(q[3:8], kp, vp, tables[:1], clens[:1], [5])
    check_attention(got[3:8], want0, "bf16")
    want1 = ref_prefill(q[8:18], kp, vp, tables[1:2], clens[1:2], [10])
    check_attention(got[8:18], want1, "bf16")


def test_max_query_len_bound(pkv):
    """max_query_len bounds every sequence's query run.  With a host query_start
    the binding rejects an undersized bound; with a device query_start the
    call covers only the last runs of a longer sequence, as the header states:
    with G = 4 runs are 32 rows from the sequence's first row, a bound of 20
    rows covers one run, so of a 70-row sequence (runs 0-31, 32-63, 64-69)
    only the last 6 rows are written."""
    import torch
    say("case prefill max_query_len bound")
    rng = np.random.default_rng(93)
    Hkv, G, D, B = 2, 4, 64, 16
    lens, qlens = (100, 30), [70, 12]
    kp, vp, tables, clens = build(rng, lens, Hkv, D, B)
    starts = np.array([0, 70, 82], np.int32)
    q = W.normal(rng, (82, Hkv * G, D), "bf16")
    out = torch.full((82, Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
    args = (out, to_dev(q), to_dev(kp), to_dev(vp), torch.from_numpy(tables).cuda(),
            torch.from_numpy(clens).cuda())
    with pytest.raises(ValueError):
        pkv.paged_attention_prefill(*args, starts, 20)
    pkv.paged_attention_prefill(*args, starts, 70)        # host query_start, bound met
    torch.cuda.synchronize()
    want = ref_prefill(q, kp, vp, tables, clens, qlens)
    check_attention(out.cpu().numpy(), want, "bf16")
    out.fill_(float("nan"))
    pkv.paged_attention_prefill(*args, torch.from_numpy(starts).cuda(), 20)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isnan(got[:64]).all()
    check_attention(got[64:], want[64:], "bf16")


@pytest.mark.parametrize("G,D,B", [(4, 128, 16), (1, 64, 32), (8, 128, 32), (2, 128, 16),
                                   (8, 128, 16), (4, 64, 16), (1, 64, 16)])
def test_prefill_fp8_matches_reference(pkv, G, D, B):
    """fp8 E4M3 pools (codes of the bf16 K/V at per-head scales; NaN codes in
    every unused slot): within the bf16 bound of the fp64 reference over the
    dequantized pools."""
    import torch
    from oracle.cache_ops import reshape_and_cache as ref_cache
    say(f"case prefill fp8 G={G} D={D} B={B}")
    rng = np.random.default_rng(950 + G * 7 + D + B)
    Hkv = 2
    k_scale = rng.uniform(0.004, 0.03, Hkv).astype(np.float32)
    v_scale = rng.uniform(0.004, 0.03, Hkv).astype(np.float32)
    N = sum(-(-L // B) for L in LENS) + 5
    bm = BlockManager(N, B, rng.permutation(N))
    ks, vs = W.pool_shapes(N, Hkv, D, B, "fp8")
    kp, vp = np.full(ks, 0x7F, np.uint8), np.full(vs, 0x7F, np.uint8)
    slots, Ks, Vs = [], [], []
    for s, L in enumerate(LENS):
        bm.add_seq(s, L)
        t = bm.tables[s]
        slots += [t[i // B] * B + i % B for i in range(L)]
        Ks.append(W.normal(rng, (L, Hkv, D), "bf16"))
        Vs.append(W.normal(rng, (L, Hkv, D), "bf16"))
    kp, vp = ref_cache(kp, vp, np.concatenate(Ks), np.concatenate(Vs), np.asarray(slots),
                       k_scale, v_scale)
    tables, clens = bm.fill_batch(range(len(LENS)), max(-(-L // B) for L in LENS))
    tables, clens = np.asarray(tables, np.int32), np.asarray(clens, np.int32)
    q = W.normal(rng, (sum(QLENS), Hkv * G, D), "bf16")
    starts = np.concatenate([[0], np.cumsum(QLENS)]).astype(np.int32)
    out = torch.full((q.shape[0], Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_attention_prefill(out, to_dev(q), to_dev(kp), to_dev(vp),
                                torch.from_numpy(tables).cuda(), torch.from_numpy(clens).cuda(),
                                torch.from_numpy(starts).cuda(), max(QLENS),
                                k_scale=torch.from_numpy(k_scale).cuda(),
                                v_scale=torch.from_numpy(v_scale).cuda())
    torch.cuda.synchronize()
    want = ref_prefill(q, kp, vp, tables, clens, QLENS, k_scale=k_scale, v_scale=v_scale)
    worst = check_attention(out.cpu().numpy(), want, "bf16")
    say(f"  worst error {worst:.3e}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_full_config(pkv, kv):
    """The benchmark's multi-token workload at full size in its launch
    configuration: 16 sequences x (1,536 cached + 512 new tokens) of the
    Llama-3-8B-shaped layer (32/8 heads, D 128, B 16), each sequence on a
    shuffled slice of the pool.  Every (row, head) output is within the bf16
    bound of the fp64 reference (over the dequantized pools for fp8)."""
    import torch
    say(f"case prefill full size {kv}")
    rng = np.random.default_rng(2100 + (kv == "fp8"))
    Hq, Hkv, D, B, S, prefix, chunk = 32, 8, 128, 16, 16, 1536, 512
    L = prefix + chunk
    nb = L // B
    N = S * nb
    ks, vs = W.pool_shapes(N, Hkv, D, B, kv)
    extra, scales = {}, {}
    if kv == "fp8":
        def codes(shape):   # finite E4M3 codes below 4 in magnitude, random sign
            return (rng.integers(0, 0x50, shape, dtype=np.uint8)
                    | (rng.integers(0, 2, shape, dtype=np.uint8) << 7))
        kp, vp = codes(ks), codes(vs)
        scales = {"k_scale": np.linspace(0.02, 0.03, Hkv).astype(np.float32),
                  "v_scale": np.linspace(0.03, 0.02, Hkv).astype(np.float32)}
        extra = {k: torch.from_numpy(v).cuda() for k, v in scales.items()}
    else:
        kp, vp = W.normal(rng, ks, "bf16"), W.normal(rng, vs, "bf16")
    tables = rng.permutation(N).astype(np.int32).reshape(S, nb)
    clens = np.full(S, L, np.int32)
    qlens = [chunk] * S
    T = S * chunk
    q = W.normal(rng, (T, Hq, D), "bf16")
    starts = (np.arange(S + 1) * chunk).astype(np.int32)
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_attention_prefill(out, to_dev(q), to_dev(kp), to_dev(vp),
                                torch.from_numpy(tables).cuda(), torch.from_numpy(clens).cuda(),
                                torch.from_numpy(starts).cuda(), chunk, **extra)
    torch.cuda.synchronize()
    say("  device done")
    want = ref_prefill(q, kp, vp, tables, clens, qlens, **scales)
    worst = check_attention(out.cpu().numpy(), want, "bf16")
    say(f"  worst error {worst:.3e} over all {T * Hq} rows")


@pytest.mark.parametrize("kv,B,lens", [("bf16", 16, (4500, 2100, 33)),
                                       ("bf16", 32, (8500, 4200, 40)),
                                       ("fp8", 16, (4500, 2100, 33))])
def test_prefill_long_contexts_cross_table_windows(pkv, kv, B, lens):
    """Contexts of more than 128 blocks: each wave reads block ids through a
    window of 128 table entries and reloads it when a tile's blocks pass its
    end (two reloads at 4,500 tokens of B = 16 and at 8,500 of B = 32, one at
    2,100 / 4,200).  The last rows of each context and a whole short prompt,
    over a shuffled NaN pool, are within the bf16 bound of the fp64
    reference."""
    import torch
    from oracle.cache_ops import reshape_and_cache as ref_cache
    say(f"case prefill long contexts {kv} B={B} lens={lens}")
    rng = np.random.default_rng(3300 + B + (kv == "fp8"))
    Hkv, G, D = 2, 4, 128
    qlens = [70, 40, lens[2]]
    extra, scales = {}, {}
    if kv == "fp8":
        scales = {"k_scale": rng.uniform(0.004, 0.03, Hkv).astype(np.float32),
                  "v_scale": rng.uniform(0.004, 0.03, Hkv).astype(np.float32)}
        N = sum(-(-L // B) for L in lens) + 5
        bm = BlockManager(N, B, rng.permutation(N))
        ks, vs = W.pool_shapes(N, Hkv, D, B, "fp8")
        kp, vp = np.full(ks, 0x7F, np.uint8), np.full(vs, 0x7F, np.uint8)
        slots, Ks, Vs = [], [], []
        for s, L in enumerate(lens):
            bm.add_seq(s, L)
            t = bm.tables[s]
            slots += [t[i // B] * B + i % B for i in range(L)]
            Ks.append(W.normal(rng, (L, Hkv, D), "bf16"))
            Vs.append(W.normal(rng, (L, Hkv, D), "bf16"))
        kp, vp = ref_cache(kp, vp, np.concatenate(Ks), np.concatenate(Vs), np.asarray(slots),
                           scales["k_scale"], scales["v_scale"])
        tables, clens = bm.fill_batch(range(len(lens)), max(-(-L // B) for L in lens))
        tables, clens = np.asarray(tables, np.int32), np.asarray(clens, np.int32)
        extra = {k: torch.from_numpy(v).cuda() for k, v in scales.items()}
    else:
        kp, vp, tables, clens = build(rng, lens, Hkv, D, B)
    assert tables.shape[1] > 2 * 128  # the longest walk passes two window ends
    q = W.normal(rng, (sum(qlens), Hkv * G, D), "bf16")
    starts = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    out = torch.full((q.shape[0], Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_attention_prefill(out, to_dev(q), to_dev(kp), to_dev(vp),
                                torch.from_numpy(tables).cuda(), torch.from_numpy(clens).cuda(),
                                torch.from_numpy(starts).cuda(), max(qlens), **extra)
    torch.cuda.synchronize()
    want = ref_prefill(q, kp, vp, tables, clens, qlens, **scales)
    worst = check_attention(out.cpu().numpy(), want, "bf16")
    say(f"  worst error {worst:.3e}")
