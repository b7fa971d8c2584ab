"""Pins for the oracle's block-pool model: the guide's worked example, hand-traced
scenarios, the beam-sharing closed form and invariants under random operation
sequences."""

import json
import os

import numpy as np
import pytest

import workloads as wl
from oracle import allocator as al
from oracle import closed_forms as cf
from oracle import run as orun


def check_invariants(pool: al.BlockPool):
    for on_host, refcount, free, n in ((False, pool.refcount, pool.free_list(), pool.num_blocks),
                                       (True, pool.host_refcount, pool.host_free_list(), pool.host_blocks)):
        live = [b for s in pool.seqs.values() if s.on_host == on_host for b in s.table]
        assert sum(refcount) == len(live)
        counts = np.bincount(np.asarray(live, dtype=np.int64), minlength=n) if live else np.zeros(n, np.int64)
        assert list(counts) == refcount
        assert len(set(free)) == len(free)
        assert all(refcount[b] == 0 for b in free)
        used = sum(1 for r in refcount if r > 0)
        assert len(free) + used == n
    for s in pool.seqs.values():
        assert len(s.table) == cf.blocks_for(s.length, pool.block_size)


def test_worked_example_blocks(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        g = json.load(f)
    for row in g["paged"]:
        pool = al.BlockPool(128, row["block_size"])
        ids = [pool.create() for _ in g["lengths"]]
        pool.append(ids, g["lengths"])
        st = pool.stats()
        assert st["logical_tokens"] == g["used_slots"]
        assert st["allocated_slots"] == row["allocated_slots"]
        assert st["used_blocks"] == row["allocated_slots"] // row["block_size"]
        check_invariants(pool)


def test_fifo_slots_by_hand():
    pool = al.BlockPool(6, 4)
    a, b = pool.create(), pool.create()
    slots, pairs = pool.append([a, b], [5, 2])
    # a takes blocks 0 then 1 (positions 0-3 -> slots 0-3, position 4 -> slot 4); b takes block 2.
    assert list(slots) == [0, 1, 2, 3, 4, 8, 9]
    assert pairs.shape == (0, 2)
    assert pool.table(a) == [0, 1] and pool.table(b) == [2]
    pool.free_seq(a)
    # freed blocks join the tail in logical order: queue is now 3, 4, 5, 0, 1
    assert pool.free_list() == [3, 4, 5, 0, 1]
    c = pool.create()
    slots, _ = pool.append([c], [6])
    assert pool.table(c) == [3, 4]
    assert list(slots) == [12, 13, 14, 15, 16, 17]


def test_fork_and_copy_on_write_by_hand():
    pool = al.BlockPool(8, 16)
    p = pool.create()
    pool.append([p], [40])  # blocks 0, 1, 2; block 2 holds 8 tokens
    c = pool.fork(p)
    assert [pool.refcount[i] for i in range(3)] == [2, 2, 2]
    slots, pairs = pool.append([c], [1])
    # the child writes into shared partial block 2 -> copy to the next free block (3)
    assert pairs.tolist() == [[2, 3]]
    assert pool.table(c) == [0, 1, 3]
    assert list(slots) == [3 * 16 + 8]
    assert pool.refcount[:4] == [2, 2, 1, 1]
    # the parent is now the last holder of block 2 and writes in place
    slots, pairs = pool.append([p], [1])
    assert pairs.shape == (0, 2) and list(slots) == [2 * 16 + 8]
    # a full shared block is never copied: fork at a block boundary
    q = pool.create()
    pool.append([q], [32])  # blocks 4, 5 full
    r = pool.fork(q)
    slots, pairs = pool.append([r], [1])
    assert pairs.shape == (0, 2)
    assert pool.table(r) == [4, 5, 6] and list(slots) == [6 * 16]
    check_invariants(pool)


def test_free_order_after_fork_free():
    pool = al.BlockPool(4, 2)
    p = pool.create()
    pool.append([p], [3])  # blocks 0, 1
    c = pool.fork(p)
    pool.free_seq(p)  # counts drop to 1: nothing reclaimed
    assert pool.free_list() == [2, 3]
    pool.free_seq(c)
    assert pool.free_list() == [2, 3, 0, 1]
    check_invariants(pool)


def test_out_of_blocks_changes_nothing():
    pool = al.BlockPool(5, 4)
    a, b = pool.create(), pool.create()
    pool.append([a, b], [6, 3])  # a: 2 blocks, b: 1 block -> 2 free
    c = pool.fork(a)
    before = (pool.free_list(), list(pool.refcount), pool.table(a), pool.table(b), pool.table(c),
              pool.length(a), pool.length(b), pool.length(c))
    # c needs a copy of a's partial block (1) + b needs 1 + a needs 1 more block: 3 > 2 free
    with pytest.raises(al.OutOfBlocks):
        pool.append([c, b, a], [3, 2, 3])
    after = (pool.free_list(), list(pool.refcount), pool.table(a), pool.table(b), pool.table(c),
             pool.length(a), pool.length(b), pool.length(c))
    assert before == after
    check_invariants(pool)


def test_argument_errors():
    pool = al.BlockPool(4, 4)
    a = pool.create()
    with pytest.raises(al.InvalidArg):
        pool.append([a, a], [1, 1])
    with pytest.raises(al.InvalidArg):
        pool.append([a], [-1])
    with pytest.raises(al.NoSuchSeq):
        pool.append([7], [1])
    with pytest.raises(al.NoSuchSeq):
        pool.free_seq(7)
    with pytest.raises(al.InvalidArg):
        al.BlockPool(3, 4, free_order=[0, 0, 1])


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(123)
    for trial in range(20):
        nb = int(rng.integers(4, 40))
        pool = al.BlockPool(nb, int(rng.choice([1, 2, 4, 16])), rng.permutation(nb))
        live = []
        for _ in range(60):
            op = rng.integers(0, 4)
            if op == 0 or not live:
                live.append(pool.create())
            elif op == 1:
                live.append(pool.fork(int(rng.choice(live))))
            elif op == 2:
                sid = int(rng.choice(live))
                pool.free_seq(sid)
                live.remove(sid)
            else:
                k = int(rng.integers(1, len(live) + 1))
                seqs = list(rng.choice(live, size=k, replace=False))
                counts = list(rng.integers(0, 20, size=k))
                snap = (pool.free_list(), list(pool.refcount))
                try:
                    slots, pairs = pool.append(seqs, counts)
                    assert len(slots) == sum(counts)
                    assert len(set(slots.tolist())) == len(slots)
                except al.OutOfBlocks:
                    assert (pool.free_list(), list(pool.refcount)) == snap
            check_invariants(pool)


def test_beam_sharing_closed_form():
    w = wl.named("beam_cow_bf16", seed=0)
    rp = orun.replay(w, with_cache=False)
    s = w.spec
    B = s.block_size
    full_prefix = s.prefix_len // B  # 62 full shared blocks
    assert s.prefix_len % B != 0
    expected_unique = 0
    for p in range(s.prompts):
        expected_unique += full_prefix + sum(cf.blocks_for(s.prefix_len + int(t), B) - full_prefix
                                             for t in w.tail_lens[p])
    st = rp.pool.stats()
    assert st["used_blocks"] == expected_unique
    private = sum(cf.blocks_for(int(n), B) for n in w.context_lens)
    assert private - expected_unique == s.prompts * (s.beams - 1) * full_prefix
    # copy-on-write fires once per beam that is not the last holder of the partial prompt block
    all_pairs = np.concatenate(rp.pairs)
    assert len(all_pairs) == s.prompts * (s.beams - 1) == 96
    assert st["sum_refcount"] == st["logical_blocks"]
    # the 62 full prompt blocks of every prompt are held by all 4 beams
    for p in range(s.prompts):
        t0 = rp.pool.table(p * s.beams)
        assert all(rp.pool.refcount[b] == s.beams for b in t0[:full_prefix])
    check_invariants(rp.pool)


def test_full_pool_long_context():
    w = wl.named("long_bf16", seed=0)
    rp = orun.replay(w, with_cache=False)
    st = rp.pool.stats()
    assert st["free_blocks"] == 0 and st["used_blocks"] == 16384
    with pytest.raises(al.OutOfBlocks):
        rp.pool.append([0], [1])


def swap_scenario():
    """The hand-traced swapping scenario (see test_swap_by_hand); returns the pool and the ids."""
    pool = al.BlockPool(6, 4, host_blocks=4)
    a = pool.create()
    pool.append([a], [6])  # device blocks 0, 1
    b = pool.fork(a)
    _, cow = pool.append([b], [1])  # b writes into shared partial block 1: copied to block 2
    c = pool.create()
    pool.append([c], [4])  # block 3
    return pool, a, b, c, cow


def test_swap_by_hand():
    pool, a, b, c, cow = swap_scenario()
    assert cow.tolist() == [[1, 2]]
    assert pool.table(a) == [0, 1] and pool.table(b) == [0, 2] and pool.table(c) == [3]
    assert pool.free_list() == [4, 5]
    # c alone: its block 3 takes host block 0 and joins the device queue's tail
    assert pool.swap_out([c]).tolist() == [[3, 0]]
    assert pool.free_list() == [4, 5, 3] and pool.table(c) == [0] and pool.on_host(c)
    # a without b is not a whole sharing group (block 0 is held by both)
    with pytest.raises(al.InvalidArg):
        pool.swap_out([a])
    # a then b: blocks met in order 0, 1, 2 take host blocks 1, 2, 3; block 0 keeps its count of 2
    assert pool.swap_out([a, b]).tolist() == [[0, 1], [1, 2], [2, 3]]
    assert pool.table(a) == [1, 2] and pool.table(b) == [1, 3]
    assert pool.host_refcount == [1, 2, 1, 1] and pool.refcount == [0] * 6
    assert pool.free_list() == [4, 5, 3, 0, 1, 2] and pool.host_free_list() == []
    # b listed first: host blocks met in order 1, 3, 2 take device blocks 4, 5, 3
    assert pool.swap_in([b, a]).tolist() == [[1, 4], [3, 5], [2, 3]]
    assert pool.table(b) == [4, 5] and pool.table(a) == [4, 3]
    assert pool.refcount[3:6] == [1, 2, 1] and pool.host_refcount == [1, 0, 0, 0]
    assert pool.host_free_list() == [1, 3, 2] and pool.free_list() == [0, 1, 2]
    assert pool.swap_in([c]).tolist() == [[0, 0]]
    assert pool.table(c) == [0] and pool.host_free_list() == [1, 3, 2, 0] and pool.free_list() == [1, 2]
    # the swapped-in sequences append as before: a's partial block 3 is its own, b's block 5 too
    slots, pairs = pool.append([a, b], [1, 1])
    assert pairs.shape == (0, 2) and list(slots) == [3 * 4 + 2, 5 * 4 + 3]
    check_invariants(pool)


def test_swap_errors_change_nothing():
    pool, a, b, c, _ = swap_scenario()
    snap = lambda: (pool.free_list(), pool.host_free_list(), list(pool.refcount), list(pool.host_refcount),
                    [pool.table(x) for x in (a, b, c)], [pool.on_host(x) for x in (a, b, c)])
    before = snap()
    with pytest.raises(al.InvalidArg):
        pool.swap_out([a])  # block 0 also held by b
    with pytest.raises(al.InvalidArg):
        pool.swap_out([c, c])
    with pytest.raises(al.NoSuchSeq):
        pool.swap_out([9])
    with pytest.raises(al.WrongTier):
        pool.swap_in([c])  # not swapped out
    small = al.BlockPool(6, 4, host_blocks=2)
    x = small.create()
    small.append([x], [9])  # 3 blocks > 2 host blocks
    with pytest.raises(al.OutOfBlocks):
        small.swap_out([x])
    assert small.table(x) == [0, 1, 2] and not small.on_host(x)
    assert snap() == before
    pool.swap_out([c])
    with pytest.raises(al.WrongTier):
        pool.swap_out([c])
    with pytest.raises(al.WrongTier):
        pool.append([c], [1])
    with pytest.raises(al.WrongTier):
        pool.fork(c)
    with pytest.raises(al.WrongTier):
        pool.block_tables([c], 4)
    # freeing a swapped-out sequence returns its host blocks
    pool.free_seq(c)
    assert pool.host_free_list() == [1, 2, 3, 0]
    check_invariants(pool)


def test_swap_round_trip_keeps_every_token():
    # brute force: distinct values per device slot, swap a group out, let other
    # sequences overwrite the freed blocks, swap it back and read every token
    from oracle import cache as oc
    rng = np.random.default_rng(5)
    B, H, d = 4, 2, 64
    pool = al.BlockPool(12, B, rng.permutation(12), host_blocks=8)
    kc, vc = oc.empty_caches(12, H, B, d, "f32")
    hk, hv = oc.empty_caches(8, H, B, d, "f32")
    p = pool.create()
    slots, _ = pool.append([p], [10])
    kv = rng.standard_normal((2, 10, H, d)).astype(np.float32)
    oc.scatter(kc, vc, kv[0], kv[1], slots)
    kids = [pool.fork(p) for _ in range(2)]
    toks = {p: (kv[0], kv[1])}
    for kid in kids:  # each child adds 3 tokens: copy-on-write of the shared partial block first
        slots, pairs = pool.append([kid], [3])
        oc.copy_blocks(kc, vc, pairs)
        new = rng.standard_normal((2, 3, H, d)).astype(np.float32)
        oc.scatter(kc, vc, new[0], new[1], slots)
        toks[kid] = (np.concatenate([kv[0], new[0]]), np.concatenate([kv[1], new[1]]))
    group = [p] + kids
    out_pairs = pool.swap_out(group)
    oc.swap_blocks(kc, vc, hk, hv, out_pairs)
    other = pool.create()
    slots, _ = pool.append([other], [4 * len(pool.free_list())])  # takes every free device block
    junk = np.full((len(slots), H, d), 7.0, np.float32)
    oc.scatter(kc, vc, junk, junk, slots)
    pool.free_seq(other)
    in_pairs = pool.swap_in(group[::-1])
    oc.swap_blocks(hk, hv, kc, vc, in_pairs)
    for sid in group:
        k, v = oc.gather(kc, vc, pool.table(sid), pool.length(sid))
        assert np.array_equal(k, toks[sid][0]) and np.array_equal(v, toks[sid][1])
    # sharing survives: the prefix blocks are still one physical block per position
    assert pool.table(p)[:2] == pool.table(kids[0])[:2] == pool.table(kids[1])[:2]
    check_invariants(pool)


def test_random_swaps_keep_invariants():
    rng = np.random.default_rng(321)
    for trial in range(20):
        nb, hb, B = int(rng.integers(4, 40)), int(rng.integers(0, 30)), int(rng.choice([1, 2, 4, 16]))
        pool = al.BlockPool(nb, B, rng.permutation(nb), host_blocks=hb)
        for _ in range(60):
            op = int(rng.integers(0, 6))
            dev = [s for s in pool.seqs if not pool.on_host(s)]
            host = [s for s in pool.seqs if pool.on_host(s)]
            total = sum(pool.refcount) + sum(pool.host_refcount)
            if op == 0 or not pool.seqs:
                pool.create()
            elif op == 1 and dev:
                pool.fork(int(rng.choice(dev)))
            elif op == 2:
                pool.free_seq(int(rng.choice(list(pool.seqs))))
            elif op == 3 and dev:
                k = int(rng.integers(1, len(dev) + 1))
                try:
                    pool.append(list(rng.choice(dev, size=k, replace=False)), list(rng.integers(0, 20, size=k)))
                except al.OutOfBlocks:
                    pass
            elif op in (4, 5):
                tier = dev if op == 4 else host
                if tier:
                    group = group_of(pool, int(rng.choice(tier)))
                    try:
                        pairs = pool.swap_out(group) if op == 4 else pool.swap_in(group)
                        assert sum(pool.refcount) + sum(pool.host_refcount) == total
                        assert len(set(pairs[:, 1].tolist())) == len(pairs)
                    except al.OutOfBlocks:
                        pass
            check_invariants(pool)


def group_of(pool: al.BlockPool, sid: int):
    """The sharing group of sid: sequences linked by a common block in the same tier."""
    group, todo = {sid}, [sid]
    while todo:
        s = pool.seqs[todo.pop()]
        for o, t in pool.seqs.items():
            if o not in group and t.on_host == s.on_host and set(t.table) & set(s.table):
                group.add(o)
                todo.append(o)
    return sorted(group)


def test_fnv1a64_published_vectors():
    # the FNV reference test vectors for the 64-bit FNV-1a hash
    assert al.fnv1a64(b"") == 0xCBF29CE484222325
    assert al.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert al.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_prefix_cache_by_hand():
    pool = al.BlockPool(8, 4)
    a = pool.create()
    slots, _ = pool.append([a], [10], token_ids=list(range(1, 11)))
    assert pool.table(a) == [0, 1, 2] and list(slots) == list(range(10))
    k0 = al.block_key(0, [1, 2, 3, 4])
    k1 = al.block_key(k0, [5, 6, 7, 8])
    assert pool.cached == {k0: 0, k1: 1}  # the partial block 2 has no key
    b, hit = pool.create_prefixed([1, 2, 3, 4, 5, 6, 7, 8, 11, 12])
    assert hit == 8 and pool.table(b) == [0, 1] and pool.refcount[:2] == [2, 2]
    slots, pairs = pool.append([b], [2], token_ids=[11, 12])
    assert pool.table(b) == [0, 1, 3] and list(slots) == [12, 13] and pairs.shape == (0, 2)
    # a prompt of exactly two blocks may take only the first: one token is always computed
    c, hit = pool.create_prefixed([1, 2, 3, 4, 5, 6, 7, 8])
    assert hit == 4 and pool.table(c) == [0] and pool.refcount[0] == 3
    pool.append([c], [4], token_ids=[5, 6, 7, 8])
    assert pool.table(c) == [0, 4] and pool.cached == {k0: 0, k1: 1}  # k1 already names block 1
    pool.free_seq(a)
    pool.free_seq(b)
    assert pool.free_list() == [5, 6, 7, 2, 1, 3]  # block 1 waits in the queue with its key
    assert pool.stats()["cached_free_blocks"] == 1
    d, hit = pool.create_prefixed([1, 2, 3, 4, 5, 6, 7, 8, 9])
    assert hit == 8 and pool.table(d) == [0, 1]
    assert pool.free_list() == [5, 6, 7, 2, 3] and pool.refcount[:2] == [2, 1]  # block 1 left the queue
    e = pool.create()
    pool.append([e], [16])  # no ids: e is not keyed
    assert pool.table(e) == [5, 6, 7, 2] and len(pool.cached) == 2
    pool.free_seq(d)
    assert pool.free_list() == [3, 1]
    f = pool.create()
    pool.append([f], [8])  # takes 3, then 1: block 1 is evicted
    assert pool.table(f) == [3, 1] and pool.cached == {k0: 0}
    g, hit = pool.create_prefixed([1, 2, 3, 4, 5, 6, 7, 8, 9])
    assert hit == 4 and pool.table(g) == [0]
    check_invariants(pool)


def test_prefix_keys_cover_the_whole_preceding_run():
    pool = al.BlockPool(16, 4)
    a = pool.create()
    pool.append([a], [13], token_ids=list(range(100, 113)))  # three full blocks
    # one token changed in block 1: blocks from there on miss
    ids = list(range(100, 113))
    ids[5] = 0
    _, hit = pool.create_prefixed(ids)
    assert hit == 4
    # block 1's tokens after a different block 0 are not the same block
    ids = [0, 0, 0, 0] + list(range(104, 113))
    _, hit = pool.create_prefixed(ids)
    assert hit == 0
    # the same prompt hits every full block it may take
    _, hit = pool.create_prefixed(list(range(100, 113)))
    assert hit == 12
    # a cached block 0 followed by tokens that are cached only after another block 0
    x = pool.create()
    pool.append([x], [9], token_ids=[7, 7, 7, 7, 8, 8, 8, 8, 1])
    _, hit = pool.create_prefixed([7, 7, 7, 7] + list(range(104, 109)))
    assert hit == 4
    check_invariants(pool)


def test_prefix_cache_refuses_hash_collisions(monkeypatch):
    monkeypatch.setattr(al, "block_key", lambda parent, tokens: 7)  # every block collides
    pool = al.BlockPool(8, 4)
    a = pool.create()
    pool.append([a], [5], token_ids=[1, 2, 3, 4, 5])
    _, hit = pool.create_prefixed([9, 9, 9, 9, 9])
    assert hit == 0  # same key, other tokens: a miss
    _, hit = pool.create_prefixed([1, 2, 3, 4, 5])
    assert hit == 4
    check_invariants(pool)


def test_prefix_cache_random_operations():
    rng = np.random.default_rng(77)
    for trial in range(15):
        B = int(rng.choice([1, 2, 4]))
        pool = al.BlockPool(int(rng.integers(8, 40)), B, host_blocks=int(rng.integers(0, 20)))
        prompts = [list(rng.integers(0, 3, size=int(rng.integers(1, 12)))) for _ in range(4)]
        for _ in range(60):
            op = int(rng.integers(0, 5))
            dev = [s for s in pool.seqs if not pool.on_host(s)]
            if op == 0 or not dev:
                ids = [int(x) for x in prompts[int(rng.integers(0, 4))]] + [int(x) for x in
                                                                           rng.integers(0, 3, size=int(rng.integers(0, 6)))]
                sid, hit = pool.create_prefixed(ids)
                assert hit % B == 0 and hit <= max(len(ids) - 1, 0)
                for i in range(hit // B):  # every reused block holds exactly this prompt's tokens
                    assert pool.block_keys[pool.table(sid)[i]][2] == tuple(ids[i * B:(i + 1) * B])
                try:
                    pool.append([sid], [len(ids) - hit], token_ids=ids[hit:])
                except al.OutOfBlocks:
                    pool.free_seq(sid)
            elif op == 1:
                pool.free_seq(int(rng.choice(list(pool.seqs))))
            elif op == 2:
                sid = int(rng.choice(dev))
                n = int(rng.integers(1, 5))
                try:
                    pool.append([sid], [n], token_ids=[int(x) for x in rng.integers(0, 3, size=n)])
                except al.OutOfBlocks:
                    pass
            elif op == 3:
                pool.fork(int(rng.choice(dev)))
            else:
                tier = [s for s in pool.seqs if pool.on_host(s) == (op == 4 and rng.random() < 0.5)]
                if tier:
                    try:
                        g = group_of(pool, int(rng.choice(tier)))
                        pool.swap_in(g) if pool.on_host(g[0]) else pool.swap_out(g)
                    except al.OutOfBlocks:
                        pass
            check_invariants(pool)
            for key, b in pool.cached.items():  # registered keys name live or queued device blocks
                assert pool.block_keys[b][0] == key
                assert pool.refcount[b] > 0 or b in pool.free


def test_freed_blocks_wait_out_every_earlier_free_block():
    """The address non-reuse window the pages ask to test: a freed block is handed out again only after every
    block that was free when it was released (FIFO), so its old contents stay addressable that long."""
    rng = np.random.default_rng(5)
    for trial in range(20):
        nb, B = int(rng.integers(8, 40)), int(rng.choice([1, 4, 16]))
        pool = al.BlockPool(nb, B, rng.permutation(nb))
        released = {}  # block -> number of blocks that must be popped before it
        pops = 0
        for _ in range(60):
            if pool.seqs and rng.random() < 0.35:
                sid = int(rng.choice(list(pool.seqs)))
                before = len(pool.free_list())
                table = pool.table(sid)
                pool.free_seq(sid)
                for i, b in enumerate(t for t in table if pool.refcount[t] == 0):
                    released[b] = pops + before + i
            else:
                sid = pool.create()
                n = int(rng.integers(1, 3 * B))
                free_before = pool.free_list()
                try:
                    pool.append([sid], [n])
                except al.OutOfBlocks:
                    pool.free_seq(sid)
                    continue
                taken = free_before[:len(free_before) - len(pool.free_list())]
                for b in taken:
                    if b in released:
                        assert pops >= released.pop(b), (b, pops)
                    pops += 1
