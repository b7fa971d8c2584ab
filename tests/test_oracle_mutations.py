"""Planted mistakes in the oracle (CPU only): every mutant must trip at least one pin.

Each mutant replaces one oracle function by a plausible wrong version (wrong head
grouping, missing scale, swapped operands, no max subtraction, off-by-one slot
offset, LIFO reuse, copy-on-write that forgets the refcount, a swap that drops
the refcount, skips the sharing-group check or releases LIFO, a block copy read
backwards) and reruns pin tests, which must then fail (an assertion, an
expected error that is not raised, or an index out of range).
"""

import numpy as np
import pytest

from oracle import allocator as al
from oracle import attention as oa
from oracle import cache as oc

import test_oracle_allocator as t_alloc
import test_oracle_attention as t_attn
import test_oracle_cache as t_cache
import test_oracle_multi as t_multi

_true_attention = oa.attention_contiguous


def _mut_head_mapping(q, k, v, scale):
    Hq, d = q.shape
    n, Hkv, _ = k.shape
    out = np.empty((Hq, d))
    for h in range(Hq):
        g = h % Hkv  # wrong: interleaved instead of contiguous groups
        s = scale * (k[:, g, :] @ q[h])
        w = np.exp(s - s.max())
        out[h] = (w @ v[:, g, :]) / w.sum()
    return out


def _mut_no_scale(q, k, v, scale):
    return _true_attention(q, k, v, 1.0)


def _mut_swap_kv(q, k, v, scale):
    return _true_attention(q, v, k, scale)


def _mut_no_max(q, k, v, scale):
    Hq, d = q.shape
    n, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.empty((Hq, d))
    with np.errstate(over="ignore", invalid="ignore"):
        for h in range(Hq):
            g = h // G
            w = np.exp(scale * (k[:, g, :] @ q[h]))
            out[h] = (w @ v[:, g, :]) / w.sum()
    return out


def _mut_drop_last_token(q, k, v, scale):
    return _true_attention(q, k[:-1] if len(k) > 1 else k, v[:-1] if len(v) > 1 else v, scale)


ATTENTION_PINS = [
    lambda: t_attn.test_matches_torch_sdpa(8, 2, 1, 16),
    lambda: t_attn.test_matches_torch_sdpa(64, 8, 300, 128),
    t_attn.test_gqa_equals_mha_with_repeated_kv,
    t_attn.test_single_token_returns_value_exactly,
    t_attn.test_dominant_key_selects_its_value,
    lambda: test_large_scores_stay_finite(),
]


def test_large_scores_stay_finite():
    # a pin in its own right: scores around 1e3 must not overflow (max subtraction)
    rng = np.random.default_rng(0)
    q = np.zeros((1, 4))
    q[0, 0] = 1.0
    k = rng.standard_normal((10, 1, 4))
    k[:, 0, 0] = 1000.0 + np.arange(10)
    v = rng.standard_normal((10, 1, 4))
    out = oa.attention_contiguous(q, k, v, 1.0)
    w = np.exp(np.arange(10) - 9.0)
    assert np.allclose(out[0], (w @ v[:, 0]) / w.sum(), atol=1e-13, rtol=0)


def _fails_some(pins):
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError, pytest.fail.Exception):
            return True
    return False


@pytest.mark.parametrize("mutant", [_mut_head_mapping, _mut_no_scale, _mut_swap_kv, _mut_no_max,
                                    _mut_drop_last_token])
def test_attention_mutants_are_caught(monkeypatch, mutant):
    assert not _fails_some(ATTENTION_PINS)  # the true oracle passes
    monkeypatch.setattr(oa, "attention_contiguous", mutant)
    assert _fails_some(ATTENTION_PINS)


def test_gather_off_by_one_is_caught(monkeypatch):
    true_gather = oc.gather

    def bad_gather(k_cache, v_cache, table, n):
        nb, H, npieces, B, X = k_cache.shape
        t = np.arange(n)
        blk = np.asarray(table)[t // B]
        off = (t + 1) % B
        return k_cache[blk, :, :, off, :].reshape(n, H, npieces * X), v_cache[blk, :, :, off]

    pins = [t_cache.test_gather_reassembles_logical_order, t_cache.test_scatter_gather_against_slot_dictionary]
    assert not _fails_some(pins)
    monkeypatch.setattr(oc, "gather", bad_gather)
    assert _fails_some(pins)
    monkeypatch.setattr(oc, "gather", true_gather)


def test_key_piece_order_is_caught(monkeypatch):
    def bad_scatter(k_cache, v_cache, k_new, v_new, slots):
        nb, H, npieces, B, X = k_cache.shape
        s = np.asarray(slots, dtype=np.int64)
        keep = s >= 0
        s = s[keep]
        # wrong: pieces reversed
        k_cache[s // B, :, :, s % B, :] = np.asarray(k_new)[keep].reshape(len(s), H, npieces, X)[:, :, ::-1, :]
        v_cache[s // B, :, :, s % B] = np.asarray(v_new)[keep]

    monkeypatch.setattr(oc, "scatter", bad_scatter)
    assert _fails_some([lambda: t_cache.test_layout_offsets("bf16", 128)])


def test_lifo_reuse_is_caught(monkeypatch):
    def lifo_free(self, sid):
        s = self._get(sid)
        for b in s.table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.appendleft(b)
        del self.seqs[sid]

    monkeypatch.setattr(al.BlockPool, "free_seq", lifo_free)
    assert _fails_some([t_alloc.test_fifo_slots_by_hand, t_alloc.test_free_order_after_fork_free])
    assert _fails_some([t_alloc.test_freed_blocks_wait_out_every_earlier_free_block])


def test_cow_without_decrement_is_caught(monkeypatch):
    def bad_append_one(self, sid, count, slots, pairs):
        B = self.block_size
        s = self._get(sid)
        if count == 0:
            return
        if s.length % B != 0 and self.refcount[s.table[-1]] > 1:
            new = self._pop()
            pairs.append((s.table[-1], new))
            s.table[-1] = new  # wrong: old block keeps its count
        for p in range(s.length, s.length + count):
            if p % B == 0:
                s.table.append(self._pop())
            slots.append(s.table[p // B] * B + p % B)
        s.length += count

    monkeypatch.setattr(al.BlockPool, "_append_one", bad_append_one)
    assert _fails_some([t_alloc.test_fork_and_copy_on_write_by_hand, t_alloc.test_beam_sharing_closed_form])


def test_cow_on_full_blocks_is_caught(monkeypatch):
    def bad_append_one(self, sid, count, slots, pairs):
        B = self.block_size
        s = self._get(sid)
        if count == 0:
            return
        if s.table and self.refcount[s.table[-1]] > 1:  # wrong: copies full blocks too
            last = s.table[-1]
            new = self._pop()
            pairs.append((last, new))
            self.refcount[last] -= 1
            s.table[-1] = new
        for p in range(s.length, s.length + count):
            if p % B == 0:
                s.table.append(self._pop())
            slots.append(s.table[p // B] * B + p % B)
        s.length += count

    monkeypatch.setattr(al.BlockPool, "_append_one", bad_append_one)
    assert _fails_some([t_alloc.test_fork_and_copy_on_write_by_hand])


def _swap_variant(carry_refcount=True, check_group=True, lifo=False):
    """A swap with one planted mistake (refcount not carried, no sharing-group check, or LIFO release)."""
    def swap(self, seqs, out):
        seqs = [int(x) for x in seqs]
        src_ref, src_q = (self.refcount, self.free) if out else (self.host_refcount, self.host_free)
        dst_ref, dst_q = (self.host_refcount, self.host_free) if out else (self.refcount, self.free)
        met, held = [], {}
        for sid in seqs:
            for b in self.seqs[sid].table:
                if b not in held:
                    held[b] = 0
                    met.append(b)
                held[b] += 1
        if check_group and any(held[b] != src_ref[b] for b in met):
            raise al.InvalidArg("not a whole group")
        if len(met) > len(dst_q):
            raise al.OutOfBlocks()
        moved = {}
        for b in met:
            nb = dst_q.popleft()
            dst_ref[nb] = src_ref[b] if carry_refcount else 1
            src_ref[b] = 0
            src_q.appendleft(b) if lifo else src_q.append(b)
            moved[b] = nb
        for sid in seqs:
            self.seqs[sid].table = [moved[b] for b in self.seqs[sid].table]
            self.seqs[sid].on_host = out
        return np.asarray([(b, moved[b]) for b in met], dtype=np.int32).reshape(-1, 2)
    return swap


@pytest.mark.parametrize("kw", [{"carry_refcount": False}, {"check_group": False}, {"lifo": True}])
def test_swap_mutants_are_caught(monkeypatch, kw):
    monkeypatch.setattr(al.BlockPool, "_swap", _swap_variant(**kw))
    assert _fails_some([t_alloc.test_swap_by_hand, t_alloc.test_swap_round_trip_keeps_every_token])


def test_swap_copy_direction_is_caught(monkeypatch):
    def reversed_pairs(src_k, src_v, dst_k, dst_v, pairs):
        for a, b in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
            dst_k[a] = src_k[b]  # wrong: pair read as (to, from)
            dst_v[a] = src_v[b]

    monkeypatch.setattr(oc, "swap_blocks", reversed_pairs)
    assert _fails_some([t_alloc.test_swap_round_trip_keeps_every_token])


def test_prefix_key_without_the_preceding_run_is_caught(monkeypatch):
    def loose_create_prefixed(self, token_ids):
        ids = [int(t) for t in token_ids]
        B = self.block_size
        sid = self.create()
        s = self.seqs[sid]
        for i in range((len(ids) - 1) // B if ids else 0):
            toks = tuple(ids[i * B:(i + 1) * B])
            hit = [b for b, (_, _, t) in self.block_keys.items() if t == toks]  # wrong: ignores what precedes
            if not hit:
                break
            b = hit[0]
            if self.refcount[b] == 0:
                self.free.remove(b)
            self.refcount[b] += 1
            s.table.append(b)
            s.length += B
        return sid, s.length

    monkeypatch.setattr(al.BlockPool, "create_prefixed", loose_create_prefixed)
    assert _fails_some([t_alloc.test_prefix_keys_cover_the_whole_preceding_run])


def test_prefix_cache_that_never_evicts_is_caught(monkeypatch):
    monkeypatch.setattr(al.BlockPool, "_forget", lambda self, b: None)
    assert _fails_some([t_alloc.test_prefix_cache_by_hand])


# -- runs of queries and rollback ---------------------------------------------------------------------

MULTI_PINS = [t_multi.test_short_runs_are_the_last_rows_of_the_whole_prompt, t_multi.test_brute_force_scalar_loops,
              t_multi.test_future_tokens_are_invisible,
              lambda: t_multi.test_whole_prompt_runs_match_torch_causal_sdpa(8, 2, 32, 16)]


def _multi_variant(shift):
    """paged_attention_multi whose query at position p sees tokens up to p + shift."""
    def multi(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, kv_dtype):
        T, Hq, d = q.shape
        out = np.full((T, Hq, d), np.nan)
        for s in range(len(query_start) - 1):
            n, qs = int(context_lens[s]), int(query_start[s + 1]) - int(query_start[s])
            k, v = oc.gather(k_cache, v_cache, block_tables[s], n)
            k, v = oc.to_f64(k, kv_dtype), oc.to_f64(v, kv_dtype)
            for i in range(qs):
                p = n - qs + i
                hi = min(max(p + 1 + shift, 1), n)
                out[int(query_start[s]) + i] = oa.attention_contiguous(oc.to_f64(q[int(query_start[s]) + i], kv_dtype),
                                                                       k[:hi], v[:hi], scale)
        return out
    return multi


@pytest.mark.parametrize("shift", [-1, 1])
def test_causal_off_by_one_is_caught(monkeypatch, shift):
    assert not _fails_some(MULTI_PINS)
    monkeypatch.setattr(oa, "paged_attention_multi", _multi_variant(shift))
    assert _fails_some(MULTI_PINS)


def test_truncate_releasing_backwards_is_caught(monkeypatch):
    def backwards(self, sid, new_len):
        s = self._on_device(sid)
        keep = -(-int(new_len) // self.block_size)
        for b in reversed(s.table[keep:]):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        s.table = s.table[:keep]
        s.length = int(new_len)
        s.tracked = False
        s.partial = []
    monkeypatch.setattr(al.BlockPool, "truncate", backwards)
    assert _fails_some([t_multi.test_truncate_by_hand])


def test_in_place_write_keeping_a_stale_key_is_caught(monkeypatch):
    def append_one(self, sid, count, slots, pairs):
        B = self.block_size
        s = self._get(sid)
        if count == 0:
            return
        if s.length % B != 0 and self.refcount[s.table[-1]] > 1:
            new = self._pop()
            pairs.append((s.table[-1], new))
            self.refcount[s.table[-1]] -= 1
            s.table[-1] = new
        for p in range(s.length, s.length + count):
            if p % B == 0:
                s.table.append(self._pop())
            slots.append(s.table[p // B] * B + p % B)
        s.length += count
    monkeypatch.setattr(al.BlockPool, "_append_one", append_one)
    assert _fails_some([t_multi.test_truncate_drops_keys_only_when_written_again])
