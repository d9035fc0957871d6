"""Seeded synthetic inputs for PagedAttention decode.

This module only draws random numbers and states request scripts; it holds no
part of the method's arithmetic (no attention, no slot or block computation).
Both the fp64 oracle (through the tests) and the HIP path consume what it
returns, so the two sides always see the same bytes.

Shapes follow the workloads the pages describe (PagedAttention: The vLLM Paper,
"Key Results": long ShareGPT-like sequences on an OPT-13B configuration; parallel
sampling that shares a prompt's blocks, "Implementation Essentials"; GQA to
shrink the KV cache, "Impact and Follow-Ups").  No dataset is read: lengths,
queries and KV values are drawn from fixed seeds.

Draw order for every workload: lengths -> initial free-block order (a seeded
permutation of the pool) -> q -> K pool -> V pool -> new-token K -> new-token V.
K/V/q values are N(0,1) in fp32; bf16 workloads round them to bf16 with
round-to-nearest-even and hand out the raw 16-bit patterns (numpy uint16).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_CHUNK = 1 << 24  # elements drawn per rng call when filling large pools


@dataclass(frozen=True)
class Config:
    """One synthetic decode workload (all sizes are per attention layer)."""

    name: str
    seed: int
    S: int            # running sequences
    Hq: int           # query heads
    Hkv: int          # KV heads
    D: int            # head dim
    B: int            # tokens per KV block
    dtype: str        # "f32" or "bf16" (q, K, V share it; output is fp32)
    kind: str         # "step" | "decode" | "steady" | "fork"
    partition_size: int = 0   # 0 = library default
    fixed_lengths: tuple = field(default=())

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


# The five workloads.  "step": prefill to L-1 tokens, then one decode step that
# appends one token per sequence (its K/V written by reshape_and_cache) and
# attends over L tokens.  "decode": the KV of all L tokens is already cached.
# "steady"/"fork": parallel sampling, 32 prompts x 8 samples sharing the
# prompt's blocks.
CONFIGS = {
    "tiny_mha_f32": Config("tiny_mha_f32", 1, S=4, Hq=4, Hkv=4, D=64, B=16, dtype="f32",
                           kind="step", fixed_lengths=(1, 15, 16, 70)),
    "opt13b_mha": Config("opt13b_mha", 2, S=64, Hq=40, Hkv=40, D=128, B=16, dtype="bf16",
                         kind="decode"),
    "llama8b_gqa": Config("llama8b_gqa", 3, S=256, Hq=32, Hkv=8, D=128, B=16, dtype="bf16",
                          kind="step", partition_size=1024),
    "sampling_steady": Config("sampling_steady", 4, S=256, Hq=32, Hkv=8, D=128, B=16,
                              dtype="bf16", kind="steady"),
    "sampling_fork": Config("sampling_fork", 4, S=256, Hq=32, Hkv=8, D=128, B=16,
                            dtype="bf16", kind="fork"),
    "long70b_b16": Config("long70b_b16", 5, S=16, Hq=64, Hkv=8, D=128, B=16, dtype="bf16",
                          kind="decode", partition_size=512),
    "long70b_b32": Config("long70b_b32", 5, S=16, Hq=64, Hkv=8, D=128, B=32, dtype="bf16",
                          kind="decode", partition_size=512),
}

PROMPTS, SAMPLES, PROMPT_LEN = 32, 8, 1024


def pool_shapes(N: int, Hkv: int, D: int, B: int, dtype: str):
    """Array shapes of the K and V pools in the library's documented layout:
    K [N, Hkv, D/x, B, x] with x elements per 16 bytes, V [N, Hkv, D, B]."""
    x = 16 // {"f32": 4, "bf16": 2, "fp8": 1}[dtype]
    return (N, Hkv, D // x, B, x), (N, Hkv, D, B)


def _rne_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = x32.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) draws in the workload dtype: float32, or bf16 bits as uint16."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = x if dtype == "f32" else _rne_bf16_bits(x)
    return out.reshape(shape)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def draw_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """Context lengths L_s after this step (the new token included)."""
    if cfg.fixed_lengths:
        return np.asarray(cfg.fixed_lengths, dtype=np.int64)
    if cfg.name == "opt13b_mha":
        return rng.integers(128, 2048, size=cfg.S, endpoint=True).astype(np.int64)
    if cfg.name == "llama8b_gqa":
        z = rng.normal(math.log(600.0), 0.8, size=cfg.S)
        return np.clip(np.rint(np.exp(z)), 16, 4096).astype(np.int64)
    if cfg.kind == "steady":
        g = rng.integers(0, 256, size=cfg.S, endpoint=True).astype(np.int64)
        return PROMPT_LEN + 1 + g
    if cfg.kind == "fork":
        r = 1 + (np.arange(PROMPTS) % 15)
        return np.repeat(PROMPT_LEN + 1 + r, SAMPLES).astype(np.int64)
    if cfg.name.startswith("long70b"):
        return np.full(cfg.S, 32768, dtype=np.int64)
    raise ValueError(cfg.name)


def script(cfg: Config, lengths: np.ndarray):
    """Request script that brings the block manager to the state before the
    decode step, and the ids that append one token in the step (in order).

    Ops: ("add", id, n) admits a sequence holding n tokens; ("fork", parent,
    child) shares the parent's blocks; ("extend", id, n) appends n tokens one at
    a time.  The step list is empty for "decode" workloads."""
    ops = []
    S = cfg.S
    if cfg.kind == "decode":
        ops = [("add", s, int(lengths[s])) for s in range(S)]
        return ops, []
    if cfg.kind == "step":
        ops = [("add", s, int(lengths[s]) - 1) for s in range(S)]
        return ops, list(range(S))
    # parallel sampling: sample i of prompt p is sequence id p*SAMPLES + i
    for p in range(PROMPTS):
        parent = p * SAMPLES
        if cfg.kind == "steady":
            ops.append(("add", parent, PROMPT_LEN))
        else:
            ops.append(("add", parent, int(lengths[parent]) - 1))
        for i in range(1, SAMPLES):
            ops.append(("fork", parent, parent + i))
    if cfg.kind == "steady":
        for s in range(S):
            g = int(lengths[s]) - 1 - PROMPT_LEN
            if g:
                ops.append(("extend", s, g))
    return ops, list(range(S))


def blocks_needed(cfg: Config, lengths: np.ndarray) -> int:
    """Distinct blocks the state after the step occupies (the pool is sized
    20% above it, rounded up)."""
    B = cfg.B
    if cfg.kind in ("decode", "step"):
        return int(sum(_ceil_div(int(L), B) for L in lengths))
    shared = PROMPTS * _ceil_div(PROMPT_LEN if cfg.kind == "steady" else int(lengths[0]) - 1, B)
    if cfg.kind == "steady":
        private = sum(_ceil_div(int(L) - PROMPT_LEN, B) for L in lengths)
        return shared + int(private)
    # fork: every sample but the last of each prompt copies the shared partial block
    return shared + PROMPTS * (SAMPLES - 1)


@dataclass
class Workload:
    cfg: Config
    lengths: np.ndarray          # int64 [S], L_s after the step
    num_blocks: int              # N
    free_order: np.ndarray       # int32 [N], initial free-queue order
    q: np.ndarray                # [S, Hq, D]
    k_pool: np.ndarray           # [N, Hkv, D/x, B, x]
    v_pool: np.ndarray           # [N, Hkv, D, B]
    k_new: np.ndarray            # [T, Hkv, D]
    v_new: np.ndarray            # [T, Hkv, D]
    ops: list
    step_ids: list

    @property
    def kv_bytes(self) -> int:
        c = self.cfg
        return int(self.lengths.sum()) * c.Hkv * c.D * 2 * c.elem_bytes


def make(name_or_cfg, *, extra_free: float = 0.2, extra_blocks: int = 0,
         pools: bool = True) -> Workload:
    """Draw one workload.  `extra_blocks` adds free blocks beyond the +20%
    (a benchmark that runs many steps needs room to grow)."""
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    rng = np.random.default_rng(cfg.seed)
    lengths = draw_lengths(cfg, rng)
    need = blocks_needed(cfg, lengths)
    N = need + math.ceil(extra_free * need) + extra_blocks
    free_order = rng.permutation(N).astype(np.int32)
    q = normal(rng, (cfg.S, cfg.Hq, cfg.D), cfg.dtype)
    ks, vs = pool_shapes(N, cfg.Hkv, cfg.D, cfg.B, cfg.dtype)
    if pools:
        k_pool = normal(rng, ks, cfg.dtype)
        v_pool = normal(rng, vs, cfg.dtype)
    else:
        k_pool = v_pool = None
    ops, step_ids = script(cfg, lengths)
    T = len(step_ids)
    k_new = normal(rng, (T, cfg.Hkv, cfg.D), cfg.dtype)
    v_new = normal(rng, (T, cfg.Hkv, cfg.D), cfg.dtype)
    return Workload(cfg, lengths, N, free_order, q, k_pool, v_pool, k_new, v_new, ops, step_ids)


def random_script(rng: np.random.Generator, n_ops: int, max_seqs: int = 8, max_add: int = 80,
                  swap: bool = False, truncate: bool = False):
    """A random block-manager op script (for state-parity tests): admissions,
    forks, single-token appends and frees over a small id space; with swap,
    also swap-outs and swap-ins (one op in five); with truncate, also
    truncations by 0 to 2*max_add/10 tokens (one op in six; the length to cut
    is drawn here, the new length is the sequence's length minus it)."""
    ops = []
    for _ in range(n_ops):
        if swap and rng.random() < 0.2:
            ops.append(("swap_out" if rng.random() < 0.5 else "swap_in",
                        int(rng.integers(0, max_seqs))))
            continue
        if truncate and rng.random() < 1 / 6:
            ops.append(("truncate_by", int(rng.integers(0, max_seqs)),
                        int(rng.integers(0, max(2, max_add // 5) + 1))))
            continue
        r = rng.random()
        sid = int(rng.integers(0, max_seqs))
        if r < 0.2:
            ops.append(("add", sid, int(rng.integers(0, max_add))))
        elif r < 0.3:
            ops.append(("fork", sid, int(rng.integers(0, max_seqs))))
        elif r < 0.85:
            ops.append(("append", sid))
        else:
            ops.append(("free", sid))
    return ops


def request_trace(rng: np.random.Generator, n: int, prompt_median: float = 256.0,
                  prompt_sigma: float = 1.0, out_median: float = 256.0, out_sigma: float = 0.8,
                  max_prompt: int = 2048, max_out: int = 1024):
    """A synthetic request trace for the continuous-batching loop: n requests
    (id, prompt_len, max_new_tokens) with log-normal prompt and output lengths
    (a long-tailed mix like chat serving traffic; not drawn from any dataset),
    all submitted at the start."""
    p = np.clip(np.rint(np.exp(rng.normal(math.log(prompt_median), prompt_sigma, n))), 1,
                max_prompt).astype(np.int64)
    o = np.clip(np.rint(np.exp(rng.normal(math.log(out_median), out_sigma, n))), 1,
                max_out).astype(np.int64)
    return [(i, int(p[i]), int(o[i])) for i in range(n)]


def prefix_trace(rng: np.random.Generator, n: int, n_prefixes: int = 4,
                 prefix_median: float = 64.0, suffix_median: float = 24.0,
                 out_median: float = 16.0, max_prefix: int = 400, max_suffix: int = 200,
                 max_out: int = 100, vocab: int = 1000):
    """Requests whose prompts start with one of a few shared prefixes (system
    prompts, few-shot templates) followed by a request-specific part; token ids
    are random and carry no meaning.  Returns [(id, prompt_len, max_new,
    token ids)], all submitted at the start."""
    lognorm = lambda med, cap: int(np.clip(np.rint(np.exp(rng.normal(math.log(med), 0.6))),
                                           1, cap))
    prefixes = [rng.integers(0, vocab, size=lognorm(prefix_median, max_prefix)).tolist()
                for _ in range(n_prefixes)]
    out = []
    for i in range(n):
        base = prefixes[int(rng.integers(0, n_prefixes))] if rng.random() < 0.85 else []
        tokens = base + rng.integers(0, vocab, size=lognorm(suffix_median, max_suffix)).tolist()
        out.append((i, len(tokens), lognorm(out_median, max_out), [int(t) for t in tokens]))
    return out
