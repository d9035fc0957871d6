"""Planted mistakes: each plausible slip in the oracle must fail some pin.

Every mutant below is a copy of an oracle function with one deliberate error
(wrong GQA head map, transposed K block, dropped scale, one token short, no
max subtraction in the softmax, slots that ignore the range start or shift the
offset, a valid-slot mask one slot too generous, LIFO free list, a CoW that
forgets to release its source, and the swap, scheduler, prefill, prefix-cache,
fp8 and truncate mutants further down).  The pins are re-run against the
mutant and at least one of them has to fail."""
import numpy as np
import pytest

import oracle.attention as oa
import oracle.block_manager as obm
import tests.test_oracle_attention as ta
import tests.test_oracle_block_manager as tb


def _mutant_decode(head_of=None, drop_scale=False, short=False):
    def decode(q, k_pool, v_pool, block_tables, context_lens, scale=None, rows=None):
        S, Hq, D = q.shape
        Hkv = k_pool.shape[1]
        G = Hq // Hkv
        if scale is None or drop_scale:
            scale = 1.0 if drop_scale else 1.0 / np.sqrt(D)
        out = np.full((S, Hq, D), np.nan)
        qf = oa.to_f64(q)
        for s in range(S):
            L = int(context_lens[s]) - (1 if short and int(context_lens[s]) > 1 else 0)
            for h in range(Hq):
                g = head_of(h, G, Hkv) if head_of else h // G
                K, V = oa.gather_kv(k_pool, v_pool, block_tables[s], L, g)
                out[s, h] = oa.attention(qf[s, h], K, V, scale)
        return out
    return decode


def _gather_transposed(k_pool, v_pool, table, L, g, k_scale=None, v_scale=None):
    N, Hkv, Dx, B, x = k_pool.shape
    D = Dx * x
    K = np.empty((L, D))
    V = np.empty((L, D))
    for j in range(-(-L // B)):
        pb, n = int(table[j]), min(B, L - j * B)
        K[j * B:j * B + n] = oa.to_f64(k_pool[pb, g].reshape(B, D)[:n])   # wrong: no transpose
        V[j * B:j * B + n] = oa.to_f64(v_pool[pb, g, :, :n].T)
    return K, V


def _attention_pins():
    ta.test_paged_equals_contiguous_sdpa("bf16", 16, 4)
    ta.test_paged_equals_contiguous_sdpa("f32", 16, 1)
    ta.test_brute_force_scalar_loops()
    ta.test_closed_forms()
    ta.test_gqa_head_map()


def _attention_no_max(q, K, V, scale):
    """softmax without subtracting the max score first (overflows on large scores)."""
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp((K @ q) * scale)
        return (p @ V) / p.sum()


def test_no_max_subtraction_fails_pins(monkeypatch):
    monkeypatch.setattr(oa, "attention", _attention_no_max)
    monkeypatch.setattr(ta, "attention", _attention_no_max)
    with pytest.raises(AssertionError):
        _attention_pins()


@pytest.mark.parametrize("mutant", ["head_mod", "no_scale", "short"])
def test_attention_mutants_fail_pins(monkeypatch, mutant):
    dec = {"head_mod": _mutant_decode(head_of=lambda h, G, Hkv: h % Hkv),
           "no_scale": _mutant_decode(drop_scale=True),
           "short": _mutant_decode(short=True)}[mutant]
    monkeypatch.setattr(ta, "paged_attention_decode", dec)
    with pytest.raises(AssertionError):
        _attention_pins()


def test_transposed_gather_fails_pins(monkeypatch):
    monkeypatch.setattr(oa, "gather_kv", _gather_transposed)
    with pytest.raises(AssertionError):
        ta.test_paged_equals_contiguous_sdpa("bf16", 16, 4)


# --- slot rule and valid-slot mask ------------------------------------------------
import tests.test_oracle_slots as tslots


def _slots_ignore_start(bm, sid, start, count):
    bm._resident(sid)
    t = bm.tables[sid]
    return [t[i // bm.B] * bm.B + i % bm.B for i in range(count)]


def _slots_offset_shift(bm, sid, start, count):
    bm._resident(sid)
    t = bm.tables[sid]
    return [t[i // bm.B] * bm.B + (i + 1) % bm.B for i in range(start, start + count)]


def _mask_one_extra(block_tables, context_lens, num_blocks, B):
    mask = np.zeros((num_blocks, B), dtype=bool)
    for table, L in zip(block_tables, context_lens):
        n = sum(1 for b in table if b >= 0)
        for t in range(min(int(L) + 1, n * B)):      # one slot past the end when there is room
            mask[int(table[t // B]), t % B] = True
    return mask


def _slot_pins():
    tslots.test_slots_on_block_pool_figure()
    for seed in range(4):
        tslots.test_slots_equal_append_history(seed)


def _mask_pins():
    tslots.test_valid_slot_mask_on_block_pool_figure()
    for seed in range(4):
        tslots.test_valid_slot_mask_counts_private_tokens(seed)


@pytest.mark.parametrize("mutant", ["ignore_start", "offset_shift"])
def test_slots_mutants_fail_pins(monkeypatch, mutant):
    fn = {"ignore_start": _slots_ignore_start, "offset_shift": _slots_offset_shift}[mutant]
    monkeypatch.setattr(tslots, "slots", fn)
    with pytest.raises(AssertionError):
        _slot_pins()


def test_generous_mask_fails_pins(monkeypatch):
    monkeypatch.setattr(tslots, "valid_slot_mask", _mask_one_extra)
    with pytest.raises(AssertionError):
        _mask_pins()


class _LifoBM(obm.BlockManager):
    def _take(self):
        b = self.free.pop()
        self.ref[b] = 1
        return b


class _LeakyCowBM(obm.BlockManager):
    def append_slot(self, sid):
        if sid not in self.tables:
            raise obm.BMError(obm.ENOSEQ)
        table, L, B = self.tables[sid], self.lens[sid], self.B
        if L % B and self.ref[table[-1]] > 1:
            if not self.free:
                raise obm.BMError(obm.ENOBLOCKS)
            dst = self._take()                  # forgets ref[src] -= 1
            src = table[-1]
            table[-1] = dst
            slot = dst * B + L % B
            self.lens[sid] = L + 1
            return slot, src, dst
        return super().append_slot(sid)


@pytest.mark.parametrize("cls", [_LifoBM, _LeakyCowBM])
def test_block_manager_mutants_fail_pins(monkeypatch, cls):
    monkeypatch.setattr(tb, "BlockManager", cls)
    failed = 0
    for pin in (tb.test_block_pool_figure, tb.test_copy_on_write_fork,
                lambda: tb.test_invariants_random_scripts(0),
                lambda: tb.test_invariants_random_scripts(1)):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0


# --- swapping -------------------------------------------------------------------
import tests.test_oracle_swap as tswap


class _SwapKeepsDeviceBlocksBM(obm.BlockManager):
    """swap_out copies to the host but never releases the device blocks."""

    def _release(self, table):
        if getattr(self, "_in_swap", False):
            return
        super()._release(table)

    def swap_out(self, sid):
        self._in_swap = True
        try:
            return super().swap_out(sid)
        finally:
            self._in_swap = False


class _SwapInReversedBM(obm.BlockManager):
    """swap_in pairs the host blocks with the new device blocks in reverse."""

    def swap_in(self, sid):
        pairs = super().swap_in(sid)
        return [(h, d) for (h, _), (_, d) in zip(pairs, reversed(pairs))]


class _LifoHostBM(obm.BlockManager):
    """Host blocks come back to the front of the host free queue."""

    def swap_in(self, sid):
        host = list(self.host_tables.get(sid, []))
        pairs = super().swap_in(sid)
        for _ in host:
            self.host_free.pop()
        self.host_free.extendleft(reversed(host))
        return pairs


@pytest.mark.parametrize("cls", [_SwapKeepsDeviceBlocksBM, _SwapInReversedBM, _LifoHostBM])
def test_swap_mutants_fail_pins(monkeypatch, cls):
    monkeypatch.setattr(tswap, "BlockManager", cls)
    failed = 0
    for pin in [tswap.test_swap_worked_example, tswap.test_swap_of_a_shared_block_keeps_the_other_owner]\
            + [lambda s=s: tswap._run_swap_script(s) for s in range(4)]:
        try:
            pin()
        except (AssertionError, obm.BMError):
            failed += 1
    assert failed > 0


# --- continuous-batching scheduler -------------------------------------------
import oracle.scheduler as osched
from tests import test_oracle_scheduler as tsched


class _SkipAheadSched(osched.Scheduler):
    """Admits a later request when the head of the queue does not fit."""

    def begin_step(self):
        if self.waiting and len(self.waiting) > 1:
            head = self.waiting[0]
            need = -(-head.ctx // self.bm.B)
            if need > self.bm.num_free():
                self.waiting.rotate(-1)
        return super().begin_step()


class _PreemptOldestSched(osched.Scheduler):
    """Preempts the oldest running request instead of the youngest."""

    def begin_step(self):
        self.running.reverse()
        out = super().begin_step()
        return out


class _NoRejoinSched(osched.Scheduler):
    """Frees finished requests only every other step (slow to let others join)."""

    def end_step(self):
        self._flip = not getattr(self, "_flip", False)
        if self._flip:
            self.in_step = False
            return
        super().end_step()


@pytest.mark.parametrize("cls", [_SkipAheadSched, _PreemptOldestSched, _NoRejoinSched])
def test_scheduler_mutants_fail_pins(monkeypatch, cls):
    monkeypatch.setattr(tsched, "Scheduler", cls)
    tests = [tsched.test_iteration_level_figure, tsched.test_preemption_drops_the_youngest_and_recomputes_it]
    tests += [lambda s=s, r=r: tsched.test_invariants_on_random_traces(s, r)
              for s in range(6) for r in (False, True)]
    failed = 0
    for t in tests:
        try:
            t()
        except (AssertionError, osched.BMError, IndexError, ValueError, KeyError):
            failed += 1
    assert failed > 0



# --- swap policy of the scheduler ---------------------------------------------
from tests import test_oracle_scheduler_swap as tss


class _SwapFreshVictimSched(osched.Scheduler):
    """Swaps out a victim admitted in the same step, whose KV is not written."""

    def _swap_victim(self, victim, fresh):
        return super()._swap_victim(victim, False)


class _AdmitWhileSwappedSched(osched.Scheduler):
    """Admits waiting requests while preempted ones are still swapped out."""

    def _may_admit(self):
        return True


class _SwapOldestSched(osched.Scheduler):
    """Preempts the oldest running request instead of the youngest."""

    def _victim(self):
        return self.running.pop(0)


@pytest.mark.parametrize("cls", [_SwapFreshVictimSched, _AdmitWhileSwappedSched,
                                 _SwapOldestSched])
def test_scheduler_swap_mutants_fail_pins(monkeypatch, cls):
    monkeypatch.setattr(tss, "Scheduler", cls)
    failed = 0
    for t in [tss.test_swap_trace_worked_by_hand, tss.test_a_victim_without_kv_is_dropped_not_swapped] + \
            [lambda s=s: tss.swap_trace_run(s, cls) for s in range(8)]:
        try:
            t()
        except (AssertionError, osched.BMError, IndexError, KeyError, ValueError):
            failed += 1
    assert failed > 0


# --- multi-token (prefill) reference -------------------------------------------
from tests import test_oracle_prefill as tp


def _mutant_prefill(shift=0, top_left=False):
    def prefill(q, k_pool, v_pool, block_tables, context_lens, query_lens, scale=None,
                rows=None):
        T, Hq, D = q.shape
        Hkv = k_pool.shape[1]
        G = Hq // Hkv
        scale = 1.0 / np.sqrt(D) if scale is None else scale
        out = np.full((T, Hq, D), np.nan)
        starts = oa.query_starts(query_lens)
        qf = oa.to_f64(q)
        for s in range(len(query_lens)):
            L, Q = int(context_lens[s]), int(query_lens[s])
            for g in range(Hkv):
                K, V = oa.gather_kv(k_pool, v_pool, block_tables[s], L, g)
                for i in range(Q):
                    p = (i if top_left else L - Q + i) + shift
                    p = max(0, min(p, L - 1))
                    for h in range(g * G, (g + 1) * G):
                        out[starts[s] + i, h] = oa.attention(qf[starts[s] + i, h], K[:p + 1],
                                                             V[:p + 1], scale)
        return out
    return prefill


@pytest.mark.parametrize("mutant", ["minus_one", "top_left"])
def test_prefill_mutants_fail_pins(monkeypatch, mutant):
    fn = _mutant_prefill(shift=-1) if mutant == "minus_one" else _mutant_prefill(top_left=True)
    monkeypatch.setattr(tp, "paged_attention_prefill", fn)
    failed = 0
    for t in (lambda: tp.test_prefill_equals_masked_sdpa("bf16", 16, 4),
              tp.test_brute_force_scalar_loops, tp.test_one_query_per_sequence_is_decode):
        try:
            t()
        except AssertionError:
            failed += 1
    assert failed > 0


# --- prefix cache ----------------------------------------------------------------
from tests import test_oracle_prefix_cache as tpc


class _NoCapBM(obm.BlockManager):
    """Lets a hit cover the whole prompt, leaving no token to compute."""

    def add_seq_prefix(self, sid, tokens, num_tokens):
        tokens = [int(t) for t in tokens]
        if self._known(sid):
            raise obm.BMError(obm.EEXIST)
        B = self.B
        hits = []
        for j in range(len(tokens) // B):
            b = self.cache.get(tuple(tokens[:(j + 1) * B]))
            if b is None:
                break
            hits.append(b)
        need = -(-num_tokens // B) - len(hits)
        if need > len(self.free) - sum(1 for b in hits if self.ref[b] == 0):
            raise obm.BMError(obm.ENOBLOCKS)
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        table = hits + [self._take() for _ in range(need)]
        self.tables[sid] = table
        self.lens[sid] = num_tokens
        return len(hits) * B


class _HitStaysFreeBM(obm.BlockManager):
    """Takes a cached block with refcount 0 without removing it from the free queue."""

    def add_seq_prefix(self, sid, tokens, num_tokens):
        free_before = list(self.free)
        cached = super().add_seq_prefix(sid, tokens, num_tokens)
        taken = [b for b in free_before if b not in self.free]
        hits = self.tables[sid][:cached // self.B]
        back = [b for b in taken if b in hits]
        self.free.extendleft(reversed(back))        # the hits stay queued
        return cached


class _StaleCacheBM(obm.BlockManager):
    """Reallocating a cached block keeps its old cache entry."""

    def _take(self):
        b = self.free.popleft()
        self.ref[b] = 1
        return b


@pytest.mark.parametrize("cls", [_NoCapBM, _HitStaysFreeBM, _StaleCacheBM])
def test_prefix_cache_mutants_fail_pins(monkeypatch, cls):
    monkeypatch.setattr(tpc, "BlockManager", cls)
    failed = 0
    for t in [tpc.test_prefix_cache_worked_example] + \
            [lambda s=s: tpc.run_prefix_script(s, cls) for s in range(6)]:
        try:
            t()
        except (AssertionError, obm.BMError, KeyError, ValueError):
            failed += 1
    assert failed > 0


# --- fp8 codec -------------------------------------------------------------------
from oracle import fp8 as ofp8
from tests import test_oracle_fp8 as tf8


def _encode_half_up(y):
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    hi = np.clip(np.searchsorted(ofp8._POS_VALS, a, side="left"), 1, len(ofp8._POS_VALS) - 1)
    lo = hi - 1
    pick_hi = (ofp8._POS_VALS[hi] - a) <= (a - ofp8._POS_VALS[lo])       # ties go up
    code = np.where(pick_hi, ofp8._POS_CODES[hi], ofp8._POS_CODES[lo]).astype(np.uint8)
    code = np.where(a >= 448.0, np.uint8(0x7E), code)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def _decode_bias8(code):
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return (-1.0 if code & 0x80 else 1.0) * m * 2.0 ** -10
    return (-1.0 if code & 0x80 else 1.0) * (1 + m / 8) * 2.0 ** (e - 8)


@pytest.mark.parametrize("mutant", ["half_up", "bias8"])
def test_fp8_mutants_fail_pins(monkeypatch, mutant):
    if mutant == "half_up":
        monkeypatch.setattr(ofp8, "encode", _encode_half_up)
        pins = [tf8.test_array_encoder_equals_the_definition]
    else:
        monkeypatch.setattr(ofp8, "e4m3_to_f64", _decode_bias8)
        pins = [lambda: tf8.test_code_points(0x38, 1.0), lambda: tf8.test_code_points(0x7E, 448.0)]
    failed = 0
    for t in pins:
        try:
            t()
        except AssertionError:
            failed += 1
    assert failed > 0


# --- truncate (speculative drafts) --------------------------------------------
from tests import test_oracle_truncate as ttr


class _TruncateKeepsCacheBM(obm.BlockManager):
    """Truncation into a cached block leaves its prefix-cache entry in place."""

    def truncate(self, sid, new_len):
        self._resident(sid)
        if new_len < 0 or new_len > self.lens[sid]:
            raise obm.BMError(obm.EINVAL)
        keep = -(-new_len // self.B)
        table = self.tables[sid]
        self._release(table[keep:])
        del table[keep:]
        self.lens[sid] = new_len


class _TruncateReversedBM(obm.BlockManager):
    """Truncation releases the cut blocks from the last one down."""

    def truncate(self, sid, new_len):
        self._resident(sid)
        if new_len < 0 or new_len > self.lens[sid]:
            raise obm.BMError(obm.EINVAL)
        table, B = self.tables[sid], self.B
        keep = -(-new_len // B)
        if new_len % B and self.ref[table[keep - 1]] == 1:
            key = self.cached_key.pop(table[keep - 1], None)
            if key is not None:
                del self.cache[key]
        self._release(list(reversed(table[keep:])))
        del table[keep:]
        self.lens[sid] = new_len


@pytest.mark.parametrize("cls", [_TruncateKeepsCacheBM, _TruncateReversedBM])
def test_truncate_mutants_fail_pins(monkeypatch, cls):
    monkeypatch.setattr(ttr, "BlockManager", cls)
    failed = 0
    for t in [ttr.test_truncate_worked_example] + \
            [lambda s=s: ttr.simulate_speculative(1600 + s, cls) for s in range(12)]:
        try:
            t()
        except (AssertionError, obm.BMError, KeyError, ValueError):
            failed += 1
    assert failed > 0
