"""Pins for the oracle's runs of queries over paged K/V (prefill, the uncached tail
of a prefix-cached prompt, speculative verification) and for rollback by
truncation.  Attention is checked against torch's causal scaled_dot_product_
attention in float64 (an independent library routine), a scalar brute force,
the decode oracle for runs of one query, and causality itself; truncation
against hand-traced queues, refcounts and copy-on-write."""

import numpy as np
import pytest
import torch

from oracle import allocator as al
from oracle import attention as oa
from oracle import cache as oc


def paged_setup(rng, lens, Hkv, d, B, kv_dtype="f32", num_blocks=None):
    """Random K/V for each sequence scattered through a shuffled FIFO pool; returns caches, tables, contiguous K/V."""
    need = sum(-(-n // B) for n in lens)
    nb = num_blocks or need + 3
    pool = al.BlockPool(nb, B, rng.permutation(nb))
    kc, vc = oc.empty_caches(nb, Hkv, B, d, kv_dtype)
    ids = [pool.create() for _ in lens]
    slots, _ = pool.append(ids, lens)
    ks = [rng.standard_normal((n, Hkv, d)).astype(np.float32) for n in lens]
    vs = [rng.standard_normal((n, Hkv, d)).astype(np.float32) for n in lens]
    oc.scatter(kc, vc, np.concatenate(ks), np.concatenate(vs), slots)
    tables, clens = pool.block_tables(ids, max(-(-n // B) for n in lens))
    return kc, vc, tables, clens, ks, vs


def causal_sdpa(q, k, v, scale):
    """torch SDPA (float64, CPU, is_causal) over a whole prompt: q [n][Hq][d], k and v [n][Hkv][d]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    K = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).repeat_interleave(G, dim=0)
    V = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).repeat_interleave(G, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=float(scale))
    return out.numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("Hq,Hkv,d,B", [(4, 4, 16, 4), (8, 2, 32, 16), (8, 1, 8, 32)])
def test_whole_prompt_runs_match_torch_causal_sdpa(Hq, Hkv, d, B):
    rng = np.random.default_rng(Hq + 10 * B)
    lens = [1, 37, 64, 5]
    kc, vc, tables, clens, ks, vs = paged_setup(rng, lens, Hkv, d, B)
    qs = [rng.standard_normal((n, Hq, d)).astype(np.float32) for n in lens]
    starts = np.concatenate([[0], np.cumsum(lens)])
    scale = np.float32(1 / np.sqrt(d))
    out = oa.paged_attention_multi(np.concatenate(qs), kc, vc, tables, clens, starts, scale, "f32")
    for s, n in enumerate(lens):
        ref = causal_sdpa(qs[s].astype(np.float64), ks[s].astype(np.float64), vs[s].astype(np.float64), scale)
        assert np.max(np.abs(out[starts[s]:starts[s + 1]] - ref)) < 1e-12


def test_short_runs_are_the_last_rows_of_the_whole_prompt():
    """A run of the last q positions equals those rows of the whole prompt's causal attention."""
    rng = np.random.default_rng(5)
    lens, runs = [50, 17, 33], [4, 17, 1]
    Hq, Hkv, d = 8, 2, 16
    kc, vc, tables, clens, ks, vs = paged_setup(rng, lens, Hkv, d, 16)
    full_q = [rng.standard_normal((n, Hq, d)).astype(np.float32) for n in lens]
    q = np.concatenate([fq[n - r:] for fq, n, r in zip(full_q, lens, runs)])
    starts = np.concatenate([[0], np.cumsum(runs)])
    out = oa.paged_attention_multi(q, kc, vc, tables, clens, starts, 0.25, "f32")
    for s, (n, r) in enumerate(zip(lens, runs)):
        ref = causal_sdpa(full_q[s].astype(np.float64), ks[s].astype(np.float64), vs[s].astype(np.float64), 0.25)
        assert np.max(np.abs(out[starts[s]:starts[s + 1]] - ref[n - r:])) < 1e-12


def test_runs_of_one_query_are_decode():
    rng = np.random.default_rng(6)
    lens = [1, 40, 129]
    kc, vc, tables, clens, _, _ = paged_setup(rng, lens, 2, 16, 16, kv_dtype="f32")
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    out = oa.paged_attention_multi(q, kc, vc, tables, clens, [0, 1, 2, 3], 0.3, "f32")
    ref = oa.paged_attention(q, kc, vc, tables, clens, 0.3, "f32")
    assert np.max(np.abs(out - ref)) < 1e-13


def test_brute_force_scalar_loops():
    rng = np.random.default_rng(7)
    lens, runs = [6, 3], [3, 2]
    Hq, Hkv, d = 4, 2, 4
    kc, vc, tables, clens, ks, vs = paged_setup(rng, lens, Hkv, d, 4)
    q = rng.standard_normal((sum(runs), Hq, d)).astype(np.float32)
    starts = [0, 3, 5]
    out = oa.paged_attention_multi(q, kc, vc, tables, clens, starts, 0.7, "f32")
    for s in range(2):
        for i in range(runs[s]):
            p = lens[s] - runs[s] + i
            row = starts[s] + i
            for h in range(Hq):
                g = h // (Hq // Hkv)
                w = [np.exp(0.7 * sum(float(q[row, h, j]) * float(ks[s][t, g, j]) for j in range(d))) for t in range(p + 1)]
                for j in range(d):
                    ref = sum(w[t] * float(vs[s][t, g, j]) for t in range(p + 1)) / sum(w)
                    assert abs(out[row, h, j] - ref) < 1e-12


def test_future_tokens_are_invisible():
    """Changing a token's K/V changes only the queries at or after its position."""
    rng = np.random.default_rng(8)
    lens = [40]
    kc, vc, tables, clens, _, _ = paged_setup(rng, lens, 2, 16, 16)
    q = rng.standard_normal((10, 4, 16)).astype(np.float32)
    starts = [0, 10]
    before = oa.paged_attention_multi(q, kc, vc, tables, clens, starts, 0.3, "f32")
    t = 35  # run positions are 30..39
    blk, off = tables[0][t // 16], t % 16
    kc[blk, :, :, off, :] += 1.0
    vc[blk, :, :, off] -= 2.0
    after = oa.paged_attention_multi(q, kc, vc, tables, clens, starts, 0.3, "f32")
    assert np.array_equal(before[:5], after[:5])
    assert np.all(np.abs(before[5:] - after[5:]).reshape(5, -1).max(axis=1) > 1e-6)


def test_run_longer_than_context_is_refused():
    rng = np.random.default_rng(9)
    kc, vc, tables, clens, _, _ = paged_setup(rng, [3], 1, 8, 4)
    with pytest.raises(ValueError):
        oa.paged_attention_multi(np.zeros((4, 1, 8), np.float32), kc, vc, tables, clens, [0, 4], 1.0, "f32")


# -- rollback ---------------------------------------------------------------------------------------


def test_truncate_by_hand():
    pool = al.BlockPool(8, 4)
    a = pool.create()
    pool.append([a], [10])
    assert pool.table(a) == [0, 1, 2]
    b = pool.fork(a)
    pool.truncate(b, 5)  # b keeps blocks 0, 1; block 2 drops to refcount 1 (a still holds it)
    assert pool.table(b) == [0, 1] and pool.refcount[:3] == [2, 2, 1] and pool.free_list() == [3, 4, 5, 6, 7]
    slots, pairs = pool.append([b], [1])  # block 1 is shared and now partly filled for b: copy on write
    assert pairs.tolist() == [[1, 3]] and list(slots) == [13] and pool.table(b) == [0, 3]
    pool.truncate(a, 0)  # a releases 0, 1, 2 in logical order; 0 is still held by b
    assert pool.table(a) == [] and pool.length(a) == 0 and pool.free_list() == [4, 5, 6, 7, 1, 2]
    pool.truncate(b, 4)
    assert pool.table(b) == [0] and pool.free_list() == [4, 5, 6, 7, 1, 2, 3]
    with pytest.raises(al.InvalidArg):
        pool.truncate(b, 5)
    with pytest.raises(al.InvalidArg):
        pool.truncate(b, -1)
    pool.truncate(b, 4)  # same length: nothing changes


def test_truncate_drops_keys_only_when_written_again():
    pool = al.BlockPool(6, 4)
    a = pool.create()
    pool.append([a], [8], token_ids=[1, 2, 3, 4, 5, 6, 7, 8])
    k0 = al.block_key(0, [1, 2, 3, 4])
    k1 = al.block_key(k0, [5, 6, 7, 8])
    assert pool.cached == {k0: 0, k1: 1}
    pool.truncate(a, 6)  # block 1 keeps its bytes: still findable
    assert pool.cached == {k0: 0, k1: 1}
    _, hit = pool.create_prefixed([1, 2, 3, 4, 5, 6, 7, 8, 9])
    assert hit == 8 and pool.refcount[1] == 2
    pool.append([a], [1])  # block 1 is shared: a copies it, the cached original stays
    assert pool.table(a) == [0, 2] and pool.cached == {k0: 0, k1: 1}
    c = pool.create()
    pool.append([c], [8], token_ids=[9, 9, 9, 9, 8, 8, 8, 8])
    pool.truncate(c, 5)
    assert len(pool.cached) == 4
    pool.append([c], [1])  # c is block 4's only holder: written in place, its key goes
    assert pool.table(c) == [3, 4] and len(pool.cached) == 3 and 4 not in pool.block_keys
    # a truncated sequence is no longer keyed
    pool.append([c], [2], token_ids=[8, 8])
    assert len(pool.cached) == 3


def test_truncate_random_operations_keep_invariants():
    rng = np.random.default_rng(12)
    for trial in range(10):
        B = int(rng.choice([1, 2, 4, 16]))
        pool = al.BlockPool(int(rng.integers(8, 40)), B)
        for _ in range(80):
            op = int(rng.integers(0, 5))
            dev = [s for s in pool.seqs if not pool.on_host(s)]
            if op == 0 or not dev:
                pool.create()
            elif op == 1:
                sid = int(rng.choice(dev))
                n = int(rng.integers(1, 2 * B + 2))
                try:
                    pool.append([sid], [n], token_ids=[int(x) for x in rng.integers(0, 2, size=n)])
                except al.OutOfBlocks:
                    pass
            elif op == 2:
                pool.fork(int(rng.choice(dev)))
            elif op == 3:
                sid = int(rng.choice(dev))
                pool.truncate(sid, int(rng.integers(0, pool.length(sid) + 1)))
            else:
                pool.free_seq(int(rng.choice(list(pool.seqs))))
            for s in pool.seqs.values():
                assert len(s.table) == -(-s.length // B)
            assert sum(pool.refcount) == sum(len(s.table) for s in pool.seqs.values())
            assert sorted(pool.free_list() + [b for b in range(pool.num_blocks) if pool.refcount[b] > 0]) == \
                list(range(pool.num_blocks))
            for key, b in pool.cached.items():
                assert pool.block_keys[b][0] == key
