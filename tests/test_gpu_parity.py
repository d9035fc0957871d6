"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bit-exact: reshape_and_cache and copy_blocks (whole pools compared as bytes).
Attention: bf16 max abs error <= 2e-3; fp32 per-row max error <= 1e-5 of the
row's max (same rounded inputs on both sides).  Every slot that holds no token
is NaN, so any read past a sequence's end or into a free block shows up."""
import numpy as np
import pytest

import workloads as W
from tests.conftest import gpu_available
from tests.gpu_cases import Case, check_attention, say, to_dev, to_host_bits

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def ragged(name, seed, lens, Hq, Hkv, D, B, dtype, P, kind="step"):
    return W.Config(name, seed, S=len(lens), Hq=Hq, Hkv=Hkv, D=D, B=B, dtype=dtype, kind=kind,
                    partition_size=P, fixed_lengths=tuple(lens))


RAGGED_LENS = (1, 2, 15, 16, 17, 31, 32, 33, 63, 100, 511, 512, 513, 1030, 1300)

# (dtype, G, D, B, P): every compiled family, both kernels, multi-partition
KERNEL_CASES = [
    ("bf16", 1, 128, 16, 512), ("bf16", 1, 64, 32, 256), ("bf16", 2, 128, 32, 512),
    ("bf16", 4, 128, 16, 512), ("bf16", 4, 64, 16, 128), ("bf16", 8, 128, 16, 512),
    ("bf16", 8, 128, 32, 512), ("bf16", 8, 64, 32, 64), ("bf16", 4, 128, 32, 32),
    ("f32", 1, 64, 16, 512), ("f32", 2, 128, 16, 256), ("f32", 4, 64, 32, 512),
    ("f32", 8, 64, 16, 96),
]


@pytest.mark.parametrize("dtype,G,D,B,P", KERNEL_CASES)
def test_ragged_all_rows(pkv, dtype, G, D, B, P):
    Hkv = 2
    cfg = ragged(f"ragged_{dtype}_G{G}_D{D}_B{B}_P{P}", 100 + G + D + B, RAGGED_LENS, Hkv * G,
                 Hkv, D, B, dtype, P)
    say(f"case {cfg.name}")
    case = Case(pkv, W.make(cfg))
    got, kp, vp = case.run_device(pkv)
    rkp, rvp = case.oracle_pools()
    assert np.array_equal(to_host_bits(kp).view(np.uint8), rkp.view(np.uint8))
    assert np.array_equal(to_host_bits(vp).view(np.uint8), rvp.view(np.uint8))
    ref = case.oracle_out(rkp, rvp)
    worst = check_attention(got, ref, dtype)
    say(f"  worst error {worst:.3e}")


@pytest.mark.parametrize("dtype,G,B,P", [("bf16", 4, 16, 2048), ("bf16", 8, 32, 4096),
                                         ("bf16", 8, 16, 1536), ("f32", 1, 16, 2048),
                                         ("bf16", 2, 32, 3072)])
def test_partitions_beyond_one_table_register(pkv, dtype, G, B, P):
    """Partitions of more than 64 blocks take their block ids from the table
    window's second register (lanes hold blocks base + l and base + 64 + l):
    every row on lengths around and across those partitions, planned and not."""
    lens = (1, 1000, 1040, P - 1, P, P + 1, 2 * P + 37, 3000)
    cfg = ragged(f"wide_{dtype}_G{G}_B{B}_P{P}", 1500 + G + B + P, lens, 2 * G, 2, 128, B, dtype,
                 P, kind="decode")
    say(f"case {cfg.name}")
    case = Case(pkv, W.make(cfg))
    ref = case.oracle_out(case.k_pool, case.v_pool)
    for plan in (False, True):
        got, _, _ = case.run_device(pkv, plan=plan)
        worst = check_attention(got, ref, dtype)
        say(f"  plan={plan}: worst error {worst:.3e}")


@pytest.mark.parametrize("dtype,G,B", [("bf16", 8, 16), ("bf16", 4, 32), ("bf16", 1, 16),
                                       ("f32", 2, 32)])
def test_load_policy_does_not_change_results(pkv, dtype, G, B):
    """PKV_ATTN_SHARED_KV only switches nontemporal loads to cached ones: the
    output must be bit-identical either way."""
    cfg = ragged(f"policy_{dtype}_G{G}_B{B}", 300 + G + B, RAGGED_LENS, 2 * G, 2, 128, B, dtype,
                 256)
    say(f"case {cfg.name}")
    case = Case(pkv, W.make(cfg))
    a, _, _ = case.run_device(pkv, shared_kv=False)
    b, _, _ = case.run_device(pkv, shared_kv=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    check_attention(a, case.oracle_out(*case.oracle_pools()), dtype)


@pytest.mark.parametrize("dtype,G,D,B,P", KERNEL_CASES[::2])
def test_plan_matches_unplanned(pkv, dtype, G, D, B, P):
    """A host work plan changes which waves run, not what they compute: the
    output is bit-identical to the unplanned launch (zero-length rows included)."""
    lens = RAGGED_LENS + (0, 3)
    cfg = ragged(f"plan_{dtype}_G{G}_D{D}_B{B}_P{P}", 400 + G + D + B, lens, 2 * G, 2, D, B,
                 dtype, P, kind="decode")
    say(f"case {cfg.name}")
    case = Case(pkv, W.make(cfg))
    a, _, _ = case.run_device(pkv, plan=False)
    b, _, _ = case.run_device(pkv, plan=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.all(b[len(RAGGED_LENS)] == 0.0)
    rows = [(s, h) for s in range(len(lens)) if lens[s] > 0 for h in range(2 * G)]
    check_attention(b, case.oracle_out(case.k_pool, case.v_pool, rows), dtype, rows)


@pytest.mark.parametrize("dtype,G,D,B,P", KERNEL_CASES)
def test_append_matches_separate_cache_write(pkv, dtype, G, D, B, P):
    """A decode step that lets the attention launch write each sequence's new
    token gives the same pools and the same output, bit for bit, as
    reshape_and_cache followed by attention."""
    Hkv = 2
    cfg = ragged(f"append_{dtype}_G{G}_D{D}_B{B}_P{P}", 500 + G + D + B, RAGGED_LENS, Hkv * G,
                 Hkv, D, B, dtype, P)
    say(f"case {cfg.name}")
    case = Case(pkv, W.make(cfg))
    a, ka, va = case.run_device(pkv, plan=True)
    b, kb, vb = case.run_device(pkv, plan=True, append=True)
    assert np.array_equal(to_host_bits(ka).view(np.uint8), to_host_bits(kb).view(np.uint8))
    assert np.array_equal(to_host_bits(va).view(np.uint8), to_host_bits(vb).view(np.uint8))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c, _, _ = case.run_device(pkv, plan=False, append=True)
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


def test_tiny_mha_config(pkv):
    """Four sequences of 1, 15, 16 and 70 tokens, fp32, with the step's
    reshape_and_cache of 4 new tokens at positions 0, 14, 15 and 69."""
    say("case tiny_mha_f32")
    case = Case(pkv, W.make("tiny_mha_f32"))
    assert [int(s) % 16 for s in case.slots] == [0, 14, 15, 69 % 16]
    got, kp, vp = case.run_device(pkv)
    rkp, rvp = case.oracle_pools()
    assert np.array_equal(to_host_bits(kp).view(np.uint8), rkp.view(np.uint8))
    assert np.array_equal(to_host_bits(vp).view(np.uint8), rvp.view(np.uint8))
    check_attention(got, case.oracle_out(rkp, rvp), "f32")


def test_empty_and_degenerate(pkv):
    """Zero-length sequences give zero rows; one-token sequences return V[0]."""
    import torch
    cfg = ragged("zero_len", 7, (0, 1, 0, 40, 1), 8, 2, 128, 16, "bf16", 0, kind="decode")
    say("case zero_len")
    case = Case(pkv, W.make(cfg))
    got, kp, vp = case.run_device(pkv)
    assert np.all(got[[0, 2]] == 0.0)
    rows = [(s, h) for s in (1, 3, 4) for h in range(8)]
    check_attention(got, case.oracle_out(case.k_pool, case.v_pool, rows), "bf16", rows)
    # an empty batch is a no-op
    out = torch.empty(0, 8, 128, dtype=torch.float32, device="cuda")
    q = torch.empty(0, 8, 128, dtype=torch.bfloat16, device="cuda")
    t = torch.empty(0, 4, dtype=torch.int32, device="cuda")
    l = torch.empty(0, dtype=torch.int32, device="cuda")
    pkv.paged_attention_decode(out, q, kp, vp, t, l, 0)
    torch.cuda.synchronize()


def test_reject_bad_calls_without_launch(pkv):
    import torch
    cfg = ragged("reject", 8, (5, 9), 8, 2, 128, 16, "bf16", 0, kind="decode")
    case = Case(pkv, W.make(cfg))
    kp, vp = to_dev(case.k_pool), to_dev(case.v_pool)
    out = torch.empty(2, 8, 128, dtype=torch.float32, device="cuda")
    q = to_dev(case.w.q)
    wide = np.full((2, 64), -1, np.int32)
    wide[:, :case.tables.shape[1]] = case.tables
    t = torch.from_numpy(wide).cuda()
    l = torch.from_numpy(case.lens).cuda()
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode(out, q, kp, vp, t, l, 1024, partition_size=512)
    assert e.value.code == pkv.PKV_EINVAL          # needs a workspace
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode(out, q, kp, vp, t, l, 9, partition_size=40)
    assert e.value.code == pkv.PKV_EINVAL


@pytest.mark.parametrize("name", ["llama8b_gqa", "sampling_fork", "sampling_steady",
                                  "opt13b_mha", "long70b_b16", "long70b_b32"])
def test_full_config(pkv, name):
    """Full-size workload in the benchmark's launch configuration (host work
    plan, load policy from the batch's sharing, the step's tokens written by the
    attention launch): the oracle's block manager reproduces the product's
    tables, slots and copy pairs; whole pools are compared bit for bit after the
    step's cache writes, and every (sequence, query head) row of the attention
    output against the fp64 oracle."""
    say(f"case {name} (full size)")
    case = Case(pkv, W.make(name))
    got, kp, vp = case.run_device(pkv, plan=True, append=len(case.slots) > 0)
    say("  device done")
    assert np.isfinite(got).all()
    if len(case.slots) or len(case.pairs):
        rkp, rvp = case.oracle_pools()
        assert np.array_equal(to_host_bits(kp).view(np.uint8), rkp.view(np.uint8))
        assert np.array_equal(to_host_bits(vp).view(np.uint8), rvp.view(np.uint8))
        say("  pools bit-exact")
    else:
        rkp, rvp = case.k_pool, case.v_pool
    worst = check_attention(got, case.oracle_out(rkp, rvp), case.w.cfg.dtype)
    c = case.w.cfg
    say(f"  all {c.S * c.Hq} rows, worst error {worst:.3e}")
    if name == "sampling_fork":
        assert len(case.pairs) == 224


@pytest.mark.parametrize("dtype,G,B,plan", [("bf16", 4, 16, True), ("bf16", 8, 32, False),
                                            ("bf16", 1, 16, True), ("f32", 2, 16, False)])
def test_merge_in_launch_over_many_launches(pkv, dtype, G, B, plan):
    """Split sequences merged inside the main launch (at most 16 partitions of
    64 tokens here): 12 launches on one workspace, alternating two batches of
    different lengths; before every launch the partials region is filled with
    NaN (so a merge that read a partial its writer had not yet made visible, or
    a stale copy in a cache, would put NaN in the output).  Every launch
    matches the oracle on every row, and the merge counters are zero after
    each."""
    import torch
    Hkv, D, P = 2, 128, 64
    batches = []
    for k, lens in enumerate(((1, 64, 65, 200, 1024, 333, 960, 7),
                              (1000, 129, 1, 640, 64, 800, 2, 1023, 450))):
        cfg = ragged(f"merge_{dtype}_G{G}_B{B}_{k}", 1200 + 10 * k + G + B, lens, Hkv * G,
                     Hkv, D, B, dtype, P, kind="decode")
        case = Case(pkv, W.make(cfg))
        ref = case.oracle_out(case.k_pool, case.v_pool)
        batches.append((case, ref, max(lens)))
    S_max = max(len(b[0].lens) for b in batches)
    ws = pkv.attention_workspace(S_max, Hkv * G, D, 1024, P)
    cbytes = 65536                                     # the merge counters
    say(f"case merge_{dtype}_G{G}_B{B} plan={plan}")
    worst = 0.0
    for it in range(12):
        case, ref, mcl = batches[it % 2]
        c = case.w.cfg
        assert -(-mcl // P) <= 16
        ws[cbytes:].fill_(0xFF)
        kp, vp = to_dev(case.k_pool), to_dev(case.v_pool)
        out = torch.full((c.S, c.Hq, c.D), float("nan"), dtype=torch.float32, device="cuda")
        pl = pkv.make_plan(case.lens, c.Hkv, c.B, case.max_blocks, mcl, P) if plan else None
        pkv.paged_attention_decode(out, to_dev(case.w.q), kp, vp,
                                   torch.from_numpy(case.tables).cuda(),
                                   torch.from_numpy(case.lens).cuda(), mcl, partition_size=P,
                                   workspace=ws, plan=pl)
        torch.cuda.synchronize()
        assert int(ws[:cbytes].count_nonzero()) == 0, it
        worst = max(worst, check_attention(out.cpu().numpy(), ref, dtype))
    say(f"  12 launches, worst error {worst:.3e}")


@pytest.mark.parametrize("dtype,G,D", [("bf16", 4, 128), ("bf16", 1, 64), ("f32", 2, 128),
                                       ("bf16", 8, 64)])
def test_reduce_more_partitions_than_one_round(pkv, dtype, G, D):
    """Rows split into up to 125 partitions of 32 tokens: more than one round of
    the 256-thread reduce (64 partitions a round), planned and unplanned."""
    lens = (4000, 2100, 64, 1, 3333, 2049)
    cfg = ragged(f"manyparts_{dtype}_G{G}_D{D}", 900 + G + D, lens, 2 * G, 2, D, 16, dtype, 32)
    say(f"case {cfg.name}")
    case = Case(pkv, W.make(cfg))
    rkp, rvp = case.oracle_pools()
    ref = case.oracle_out(rkp, rvp)
    for plan in (False, True):
        got, _, _ = case.run_device(pkv, plan=plan)
        worst = check_attention(got, ref, dtype)
        say(f"  plan={plan}: worst error {worst:.3e}")


def test_context_beyond_table_row_is_clamped(pkv):
    """A length beyond the table row (max_blocks * B tokens) is read as the row's
    capacity: the output covers the first max_blocks * B tokens."""
    import torch
    lens = (1024, 100, 700)
    cfg = ragged("clamp", 950, lens, 8, 2, 128, 16, "bf16", 512, kind="decode")
    say("case clamp")
    case = Case(pkv, W.make(cfg))
    cap_blocks = 40                                    # 640 tokens per row
    tables = np.ascontiguousarray(case.tables[:, :cap_blocks])
    kp, vp = to_dev(case.k_pool), to_dev(case.v_pool)
    q = to_dev(case.w.q)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device="cuda")
    from oracle.attention import paged_attention_decode as ref_decode
    ref = ref_decode(case.w.q, case.k_pool, case.v_pool, tables,
                     np.minimum(np.asarray(lens, np.int32), cap_blocks * 16))
    for plan in (False, True):
        out = torch.full((3, 8, 128), float("nan"), dtype=torch.float32, device="cuda")
        ws = pkv.attention_workspace(3, 8, 128, 1024, 512, device="cuda")
        pl = pkv.make_plan(np.asarray(lens, np.int32), 2, 16, cap_blocks, 1024, 512) if plan \
            else None
        pkv.paged_attention_decode(out, q, kp, vp, torch.from_numpy(tables).cuda(), lens_dev,
                                   1024, partition_size=512, workspace=ws, plan=pl)
        torch.cuda.synchronize()
        worst = check_attention(out.cpu().numpy(), ref, "bf16")
        say(f"  plan={plan}: worst error {worst:.3e}")


@pytest.mark.parametrize("plan", [False, True])
def test_append_only_where_the_launch_covers_the_last_position(pkv, plan):
    """A step's token is written only when the launch covers the sequence's
    last position: not beyond the table row (max_blocks * B tokens), not beyond
    the partitions max_context_len sizes.  The other sequences' tokens land as
    reshape_and_cache would write them; nothing else in the pools changes."""
    import torch
    from oracle.cache_ops import reshape_and_cache as ref_cache
    lens = (100, 700, 40)
    cfg = ragged("append_cover", 960, lens, 8, 2, 128, 16, "bf16", 256)
    say(f"case append_cover plan={plan}")
    case = Case(pkv, W.make(cfg))
    assert list(case.w.step_ids) == [0, 1, 2]
    q = to_dev(case.w.q)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device="cuda")
    # (table row width in blocks, max_context_len): 32 blocks hold 512 tokens, so
    # the 700-token sequence is clamped; max_context_len 200 gives one 256-token
    # partition, which does not reach position 699 either
    for width, mcl in ((32, 700), (case.tables.shape[1], 200)):
        tables = np.ascontiguousarray(case.tables[:, :width])
        kp, vp = to_dev(case.k_pool), to_dev(case.v_pool)
        out = torch.empty((3, 8, 128), dtype=torch.float32, device="cuda")
        ws = pkv.attention_workspace(3, 8, 128, mcl, 256, device="cuda")
        pl = pkv.make_plan(np.asarray(lens, np.int32), 2, 16, width, mcl, 256) if plan else None
        pkv.paged_attention_decode(out, q, kp, vp, torch.from_numpy(tables).cuda(), lens_dev, mcl,
                                   partition_size=256, workspace=ws, plan=pl,
                                   new_key=to_dev(case.w.k_new), new_value=to_dev(case.w.v_new))
        torch.cuda.synchronize()
        keep = [0, 2]
        rk, rv = ref_cache(case.k_pool, case.v_pool, case.w.k_new[keep], case.w.v_new[keep],
                           case.slots[keep])
        assert np.array_equal(to_host_bits(kp).view(np.uint8), rk.view(np.uint8)), (width, mcl)
        assert np.array_equal(to_host_bits(vp).view(np.uint8), rv.view(np.uint8)), (width, mcl)
        rows = [(s, h) for s in keep for h in range(8)]
        check_attention(out.cpu().numpy(), case.oracle_out(rk, rv, rows), "bf16", rows)
