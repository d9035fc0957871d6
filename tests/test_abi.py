"""The C ABI library: loads, exports every declared symbol, validates on the host
(CPU only: no call here reaches a kernel launch)."""
import ctypes
import os
import re

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("pkv_paged_attention_decode", "pkv_reshape_and_cache", "pkv_copy_blocks",
                     "pkv_bm_create", "pkv_bm_fork", "pkv_bm_free_seq", "pkv_bm_append_slot",
                     "pkv_bm_refcount"):
        assert required in names


def test_library_exports_every_declared_symbol(pkv):
    lib = ctypes.CDLL(pkv.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing
    # and the binding declares a signature for each of them
    assert sorted(pkv.SIGNATURES) == declared_functions()


def test_single_hip_runtime_in_process(pkv):
    maps = open("/proc/self/maps").read()
    runtimes = set(re.findall(r"\S*libamdhip64\.so\S*", maps))
    assert len(runtimes) <= 1, runtimes


def test_host_validation_rejects_before_launch(pkv):
    lib = pkv.lib
    fake = ctypes.c_void_p(4096)            # never dereferenced: every call below fails validation
    odd = ctypes.c_void_p(4098)
    tbl = ctypes.c_void_p(4096)
    # unsupported head dim / block size / group size
    for D, B, Hq, Hkv in ((96, 16, 8, 8), (128, 8, 8, 8), (128, 16, 24, 8)):
        st = lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, Hq, Hkv, D, B, 4,
                                            8, 16, 0.1, 0, None, 0, 0, None, 0, pkv.PKV_BF16, 0, None,
                                            None, None)
        assert st == pkv.PKV_EUNSUPPORTED
    # Hq not a multiple of Hkv, bad partition size, misaligned pointer, bad dtype
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, 6, 4, 128, 16, 4,
                                          8, 16, 0.1, 0, None, 0, 0, None, 0, 1, 0, None, None, None) == pkv.PKV_EINVAL
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, 8, 8, 128, 16, 4,
                                          8, 16, 0.1, 48, None, 0, 0, None, 0, 1, 0, None, None, None) == pkv.PKV_EINVAL
    # a partition may span at most 128 blocks (4096 tokens = 256 blocks of 16)
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, 8, 8, 128, 16, 4,
                                          8, 16, 0.1, 4096, None, 0, 0, None, 0, 1, 0, None, None, None) == pkv.PKV_EINVAL
    assert lib.pkv_paged_attention_decode(odd, fake, fake, fake, None, None, tbl, tbl, 1, 8, 8, 128, 16, 4,
                                          8, 16, 0.1, 0, None, 0, 0, None, 0, 1, 0, None, None, None) == pkv.PKV_EINVAL
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, 8, 8, 128, 16, 4,
                                          8, 16, 0.1, 0, None, 0, 0, None, 0, 7, 0, None, None, None) == pkv.PKV_EINVAL
    # the score scale must be positive and finite
    for bad in (0.0, -0.1, float("inf"), float("nan")):
        assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, 8, 8, 128,
                                              16, 4, 8, 16, bad, 0, None, 0, 0, None, 0, 1, 0, None,
                                              None, None) == pkv.PKV_EINVAL
    # unknown flag bits
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, 8, 8, 128, 16, 4,
                                          8, 16, 0.1, 0, None, 0, 0, None, 0, 1, 2, None, None, None) == pkv.PKV_EINVAL
    # the step's new token needs both rows, 16-byte aligned
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, fake, None, tbl, tbl, 1, 8, 8, 128, 16, 4,
                                          8, 16, 0.1, 0, None, 0, 0, None, 0, 1, 0, None, None, None) == pkv.PKV_EINVAL
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, fake, odd, tbl, tbl, 1, 8, 8, 128, 16, 4,
                                          8, 16, 0.1, 0, None, 0, 0, None, 0, 1, 0, None, None, None) == pkv.PKV_EINVAL
    # long contexts need a workspace
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, 8, 8, 128, 16, 64,
                                          128, 1024, 0.1, 512, None, 0, 0, None, 0, 1, 0, None, None, None) == pkv.PKV_EINVAL
    # empty batches are a no-op success
    assert lib.pkv_paged_attention_decode(None, None, None, None, None, None, None, None, 0, 8, 8, 128, 16, 4,
                                          8, 16, 0.1, 0, None, 0, 0, None, 0, 1, 0, None, None, None) == pkv.PKV_OK
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 0, 8, 128, 16, 8, 1,
                                     None, None, None) == pkv.PKV_OK
    assert lib.pkv_copy_blocks(None, None, None, 0, 8, 128, 16, 8, 1, None) == pkv.PKV_OK
    assert lib.pkv_reshape_and_cache(odd, fake, fake, fake, tbl, 4, 8, 128, 16, 8, 1,
                                     None, None, None) == pkv.PKV_EINVAL
    # fp8 pools need both scales; fp8 attention needs scales and a compiled G
    assert lib.pkv_reshape_and_cache(fake, fake, fake, fake, tbl, 4, 8, 128, 16, 8, 2,
                                     None, None, None) == pkv.PKV_EINVAL
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, 48,
                                          3, 128, 16, 4, 8, 16, 0.1, 0, None, 0, 0, None, 0, 2,
                                          0, fake, fake, None) == pkv.PKV_EUNSUPPORTED   # G = 16
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, 32,
                                          8, 128, 16, 4, 8, 16, 0.1, 0, None, 0, 0, None, 0, 2,
                                          0, None, None, None) == pkv.PKV_EINVAL         # no scales
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, fake, None, tbl, tbl, 1, 32,
                                          8, 128, 16, 4, 8, 16, 0.1, 0, None, 0, 0, None, 0, 2,
                                          0, fake, fake, None) == pkv.PKV_EINVAL         # half an append
    assert lib.pkv_paged_attention_decode(fake, fake, fake, fake, None, None, tbl, tbl, 1, 32,
                                          8, 128, 16, 4, 8, 16, 0.1, 0, None, 0, 0, None, 0, 3,
                                          0, fake, fake, None) == pkv.PKV_EINVAL         # dtype 3
    assert lib.pkv_copy_blocks(fake, odd, tbl, 3, 8, 128, 16, 8, 1, None) == pkv.PKV_EINVAL


def test_swap_blocks_validation(pkv):
    """Host-side checks only: nothing here can launch (a pointer the HIP runtime
    does not know, or no GPU at all, is rejected before any launch)."""
    lib = pkv.lib
    fake, odd = ctypes.c_void_p(4096), ctypes.c_void_p(4098)
    args = lambda dk, n, dtype=1, nb=8: (dk, fake, nb, fake, fake, nb, fake, n, 8, 128, 16,
                                         dtype, None)
    assert lib.pkv_swap_blocks(*args(fake, 0)) == pkv.PKV_OK          # empty: no-op
    assert lib.pkv_swap_blocks(*args(fake, -1)) == pkv.PKV_EINVAL
    assert lib.pkv_swap_blocks(*args(fake, 1, dtype=7)) == pkv.PKV_EINVAL
    assert lib.pkv_swap_blocks(*args(fake, 1, nb=0)) == pkv.PKV_EINVAL
    assert lib.pkv_swap_blocks(*args(odd, 1)) == pkv.PKV_EINVAL         # misaligned
    # memory the runtime cannot map for the GPU (here: an address it never gave out)
    assert lib.pkv_swap_blocks(*args(fake, 1)) == pkv.PKV_EINVAL


def test_prefill_validation(pkv):
    """Host-side checks of pkv_paged_attention_prefill (nothing here launches)."""
    lib = pkv.lib
    fake = ctypes.c_void_p(4096)

    def call(S=2, T=8, Hq=8, Hkv=2, D=128, B=16, mq=4, scale=0.1, dtype=1, odd=False,
             scales=None):
        out = ctypes.c_void_p(4098) if odd else fake
        ks = vs = scales
        return lib.pkv_paged_attention_prefill(out, fake, fake, fake, fake, fake, fake, S, T, Hq,
                                               Hkv, D, B, 4, 16, mq, scale, dtype, ks, vs, None)
    assert call(dtype=0) == pkv.PKV_EUNSUPPORTED          # fp32 pools
    assert call(dtype=2) == pkv.PKV_EINVAL                # fp8 pools without scales
    assert call(dtype=2, scales=fake, D=96) == pkv.PKV_EUNSUPPORTED
    assert call(dtype=2, scales=fake, S=0) == pkv.PKV_OK
    assert call(Hq=48, Hkv=3) == pkv.PKV_EUNSUPPORTED     # G = 16
    assert call(D=96) == pkv.PKV_EUNSUPPORTED
    assert call(B=8) == pkv.PKV_EUNSUPPORTED
    assert call(Hq=6, Hkv=4) == pkv.PKV_EINVAL           # Hq not a multiple of Hkv
    assert call(scale=0.0) == pkv.PKV_EINVAL
    assert call(dtype=5) == pkv.PKV_EINVAL
    assert call(odd=True) == pkv.PKV_EINVAL               # misaligned output
    assert call(S=0) == pkv.PKV_OK and call(T=0) == pkv.PKV_OK and call(mq=0) == pkv.PKV_OK
    assert call(mq=-1) == pkv.PKV_EINVAL


def test_workspace_size_formula(pkv):
    """16384 int32 merge counters, then the partials (D + 2 floats per query
    head and partition)."""
    f = pkv.pkv_attention_workspace_bytes
    assert f(256, 32, 128, 512, 0) == 0                 # one partition: no workspace
    assert f(16, 64, 128, 32768, 512) == 65536 + 16 * 64 * 64 * 130 * 4
    assert f(4, 8, 64, 513, 512) == 65536 + 4 * 8 * 2 * 66 * 4
    assert f(0, 8, 64, 5000, 0) == 0


def test_status_strings(pkv):
    for code in range(-7, 1):
        assert pkv.lib.pkv_status_string(code).decode().startswith("PKV_")


def test_loop_create_validation(pkv):
    """pkv_loop_create rejects bad or mismatched configurations on the host,
    before it allocates anything (no HIP call reached)."""
    bm = pkv.BlockManager(32, 16)
    sched = pkv.Scheduler(bm, 4)
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(0x10000)    # never dereferenced: validation fails first

    def create(cfg, k=fake, v=fake, hk=None, hv=None, ks=None, vs=None):
        return pkv.lib.pkv_loop_create(ctypes.byref(cfg) if cfg is not None else None, bm._h,
                                       sched._h, k, v, hk, hv, ks, vs, None, ctypes.byref(h))

    def cfg(**kw):
        base = dict(num_blocks=32, block_size=16, q_heads=8, kv_heads=2, head_dim=128,
                    max_running=4, max_len=256, partition_size=0, host_blocks=0, dtype=1)
        base.update(kw)
        return pkv.LoopConfig(**base)

    EINVAL, EUNSUP = -1, -5
    assert create(None) == EINVAL
    assert create(cfg(block_size=32)) == EINVAL           # not the block manager's
    assert create(cfg(num_blocks=31)) == EINVAL
    assert create(cfg(q_heads=6, kv_heads=4)) == EINVAL   # heads do not divide
    assert create(cfg(max_running=0)) == EINVAL
    assert create(cfg(max_len=0)) == EINVAL
    assert create(cfg(partition_size=-1)) == EINVAL
    assert create(cfg(host_blocks=8)) == EINVAL           # no host pool given
    assert create(cfg(dtype=0)) == EUNSUP                 # fp32 pools: not in the loop
    assert create(cfg(dtype=7)) == EUNSUP
    assert create(cfg(dtype=2)) == EINVAL                 # fp8 without scales
    assert create(cfg(), k=None) == EINVAL
    assert h.value is None
    info = pkv.LoopStepInfo()
    src = pkv.LoopSource()
    assert pkv.lib.pkv_loop_step(None, ctypes.byref(src), ctypes.byref(info)) == EINVAL
    assert pkv.lib.pkv_loop_copy_outputs(None, None, None) == EINVAL
    pkv.lib.pkv_loop_destroy(None)
