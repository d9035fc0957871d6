"""pkv_paged_attention_decode_noalloc, the decode call for callers that cannot
allocate, against pkv_paged_attention_decode with a caller workspace, through
the C ABI: two calls in a row on the library's static scratch, the second with
a smaller batch, each bit-identical to the workspace call (output and pools)
and within the bf16 bound of the fp64 oracle.  A third call splits into more
partitions than the main launch merges, so the reduce launch reads the static
scratch too."""
import numpy as np
import pytest

import workloads as W
from tests.conftest import gpu_available
from tests.gpu_cases import Case, check_attention, say, to_dev, to_host_bits

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _call(pkv, case, P, noalloc):
    import torch
    c = case.w.cfg
    kp, vp = to_dev(case.k_pool), to_dev(case.v_pool)
    out = torch.full((c.S, c.Hq, c.D), float("nan"), dtype=torch.float32, device="cuda")
    mcl = int(case.lens.max())
    pl = pkv.make_plan(case.lens, c.Hkv, c.B, case.max_blocks, mcl, P)
    kw = dict(partition_size=P, plan=pl, new_key=to_dev(case.w.k_new),
              new_value=to_dev(case.w.v_new))
    args = (out, to_dev(case.w.q), kp, vp, torch.from_numpy(case.tables).cuda(),
            torch.from_numpy(case.lens).cuda(), mcl)
    if noalloc:
        pkv.paged_attention_decode_noalloc(*args, **kw)
    else:
        ws = pkv.attention_workspace(c.S, c.Hq, c.D, mcl, P)
        pkv.paged_attention_decode(*args, workspace=ws, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), to_host_bits(kp), to_host_bits(vp)


def test_noalloc_matches_workspace_call(pkv):
    calls = [
        # (name, seed, lengths, Hq, Hkv, B, P): a larger batch first, then a smaller one
        ("noalloc_big", 1301, (1, 17, 64, 300, 513, 1024, 1300, 1299, 700, 33, 2, 900), 16, 4,
         16, 128),
        ("noalloc_small", 1302, (5, 129, 260, 40), 16, 2, 32, 64),
        ("noalloc_reduce", 1303, (1300, 40, 999), 8, 2, 16, 32),   # 41 partitions
    ]
    for name, seed, lens, Hq, Hkv, B, P in calls:
        cfg = W.Config(name, seed, S=len(lens), Hq=Hq, Hkv=Hkv, D=128, B=B, dtype="bf16",
                       kind="step", partition_size=P, fixed_lengths=tuple(lens))
        say(f"case {name}")
        case = Case(pkv, W.make(cfg))
        got, gk, gv = _call(pkv, case, P, noalloc=True)
        want, wk, wv = _call(pkv, case, P, noalloc=False)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), name
        assert np.array_equal(gk.view(np.uint8), wk.view(np.uint8)), name
        assert np.array_equal(gv.view(np.uint8), wv.view(np.uint8)), name
        rk, rv = case.oracle_pools()
        assert np.array_equal(gk.view(np.uint8), rk.view(np.uint8)), name
        worst = check_attention(got, case.oracle_out(rk, rv), "bf16")
        say(f"  bit-identical to the workspace call, worst error {worst:.3e}")


def test_noalloc_rejects_calls_beyond_the_scratch(pkv):
    import torch
    S, Hq, Hkv, D, B, P = 64, 64, 8, 128, 16, 512
    mcl = 32768                                    # 64 partitions: 136 MB of partials
    assert pkv.attention_workspace_bytes(S, Hq, D, mcl, P) > pkv.PKV_SCRATCH_BYTES
    N = 4
    ks, vs = pkv.pool_shapes(N, Hkv, D, B, torch.bfloat16)
    kp = torch.zeros(ks, dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros(vs, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((S, Hq, D), dtype=torch.float32, device="cuda")
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros((S, mcl // B), dtype=torch.int32, device="cuda")
    lens = torch.full((S,), mcl, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode_noalloc(out, q, kp, vp, tables, lens, mcl, partition_size=P)
    assert e.value.code == pkv.PKV_ENOSCRATCH
    torch.cuda.synchronize()
    assert int(out.count_nonzero()) == 0           # nothing was launched
