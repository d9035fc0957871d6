"""The seeded generators reproduce the documented workload sizes (CPU only)."""
import numpy as np

import workloads as W
from oracle.block_manager import BlockManager, run_ops


def test_length_recipes():
    w = W.make("llama8b_gqa", pools=False)
    assert int(w.lengths.sum()) == 213551 and w.lengths.min() == 62 and w.lengths.max() == 4096
    assert w.num_blocks == 13468 + 2694
    w = W.make("opt13b_mha", pools=False)
    assert int(w.lengths.sum()) == 73505 and w.num_blocks == 4623 + 925
    assert W.make("long70b_b16", pools=False).num_blocks == 39322
    assert W.make("long70b_b32", pools=False).num_blocks == 19661


def test_scripts_fit_their_pools():
    for name in W.CONFIGS:
        if name.startswith("long70b"):
            continue
        w = W.make(name, pools=False)
        bm = BlockManager(w.num_blocks, w.cfg.B, w.free_order)
        codes, _ = run_ops(bm, w.ops)
        assert all(c == 0 for c in codes)
        pairs = []
        for sid in w.step_ids:
            slot, src, dst = bm.append_slot(sid)
            if src >= 0:
                pairs.append((src, dst))
        lens = [bm.lens[s] for s in range(w.cfg.S)]
        assert lens == w.lengths.tolist()
        if name == "sampling_fork":
            assert len(pairs) == 224
        else:
            assert not pairs
        if name == "sampling_steady":
            assert bm.num_free() == w.num_blocks - (2048 + 2252)


def test_draws_are_deterministic_bf16_rne():
    a = W.normal(np.random.default_rng(0), (1000,), "bf16")
    b = W.normal(np.random.default_rng(0), (1000,), "bf16")
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    x = np.random.default_rng(0).standard_normal(1000, dtype=np.float32)
    back = (a.astype(np.uint32) << 16).view(np.float32)
    # round to nearest: the bf16 value is within half a bf16 ulp of the fp32 draw
    ulp = np.abs(x) * 2.0 ** -7
    assert np.all(np.abs(back - x) <= 0.5 * ulp * 1.0001 + 1e-38)
