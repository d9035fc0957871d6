"""GPU: the same launch twice gives the same bits.

The attention kernels make no decision that depends on timing (the in-launch
partition merge fixes its order by partition index, and every softmax
reference is a function of the scores alone), so two launches over the same
inputs must agree bit for bit, in the output and in the pools.  A kernel that
read a register before the instruction writing it had finished (a missed
hardware wait) would break this while staying inside the error bound.
Each case launches three times and checks the outputs against the fp64 oracle
too."""
import numpy as np
import pytest

import workloads as W
from oracle.attention import paged_attention_decode as ref_decode
from tests.conftest import gpu_available
from tests.gpu_cases import Case, check_attention, say, to_dev, to_host_bits
from tests.test_gpu_fp8 import _fp8_pools, _u8
from tests.test_gpu_prefill import LENS as PF_LENS, QLENS as PF_QLENS, build, run

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

RAGGED = (1, 2, 15, 16, 17, 31, 32, 33, 63, 100, 511, 512, 513, 1030, 1300)


# (dtype, G, D, B, P, append, plan): in-launch merges, the reduce launch, both
# block sizes, the append path
@pytest.mark.parametrize("dtype,G,D,B,P,append,plan", [
    ("bf16", 4, 128, 32, 256, True, False), ("bf16", 8, 128, 16, 512, True, True),
    ("bf16", 4, 128, 16, 64, False, True), ("bf16", 8, 64, 32, 2048, True, False),
    ("f32", 2, 128, 16, 256, False, False)])
def test_decode_repeats_bit_for_bit(pkv, dtype, G, D, B, P, append, plan):
    Hkv = 2
    cfg = W.Config(f"repeat_{dtype}_G{G}_D{D}_B{B}_P{P}", 900 + G + D + B, S=len(RAGGED),
                   Hq=Hkv * G, Hkv=Hkv, D=D, B=B, dtype=dtype, kind="step", partition_size=P,
                   fixed_lengths=RAGGED)
    say(f"case {cfg.name} append={append} plan={plan}")
    case = Case(pkv, W.make(cfg))
    runs = [case.run_device(pkv, plan=plan, append=append) for _ in range(3)]
    out0, kp0, vp0 = runs[0]
    for out, kp, vp in runs[1:]:
        assert np.array_equal(out.view(np.uint32), out0.view(np.uint32))
        assert np.array_equal(to_host_bits(kp).view(np.uint8), to_host_bits(kp0).view(np.uint8))
        assert np.array_equal(to_host_bits(vp).view(np.uint8), to_host_bits(vp0).view(np.uint8))
    worst = check_attention(out0, case.oracle_out(*case.oracle_pools()), dtype)
    say(f"  3 launches identical, worst error {worst:.3e}")


@pytest.mark.parametrize("G,B,P", [(4, 16, 512), (8, 32, 96)])
def test_fp8_decode_repeats_bit_for_bit(pkv, G, B, P):
    import torch
    say(f"case fp8 repeat G={G} B={B} P={P}")
    rng = np.random.default_rng(950 + G + B + P)
    Hkv, D = 2, 128
    k_scale = rng.uniform(0.004, 0.03, Hkv).astype(np.float32)
    v_scale = rng.uniform(0.004, 0.03, Hkv).astype(np.float32)
    kp, vp, tables, clens, _ = _fp8_pools(rng, RAGGED, Hkv, D, B, k_scale, v_scale)
    S = len(RAGGED)
    q = W.normal(rng, (S, Hkv * G, D), "bf16")
    mcl = int(clens.max())
    ws = pkv.attention_workspace(S, Hkv * G, D, mcl, P, device="cuda")
    outs = []
    for _ in range(3):
        out = torch.full((S, Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
        pkv.paged_attention_decode(out, to_dev(q), _u8(kp), _u8(vp),
                                   torch.from_numpy(tables).cuda(), torch.from_numpy(clens).cuda(),
                                   mcl, partition_size=P, workspace=ws,
                                   k_scale=torch.from_numpy(k_scale).cuda(),
                                   v_scale=torch.from_numpy(v_scale).cuda())
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    want = ref_decode(q, kp, vp, tables, clens, k_scale=k_scale, v_scale=v_scale)
    worst = check_attention(outs[0], want, "bf16")
    say(f"  3 launches identical, worst error {worst:.3e}")


@pytest.mark.parametrize("G,D,B", [(4, 128, 16), (8, 128, 32)])
def test_prefill_repeats_bit_for_bit(pkv, G, D, B):
    say(f"case prefill repeat G={G} D={D} B={B}")
    rng = np.random.default_rng(970 + G + D + B)
    Hkv = 2
    kp, vp, tables, clens = build(rng, PF_LENS, Hkv, D, B)
    q = W.normal(rng, (int(sum(PF_QLENS)), Hkv * G, D), "bf16")
    outs = [run(pkv, q, kp, vp, tables, clens, PF_QLENS) for _ in range(3)]
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    say("  3 launches identical")
