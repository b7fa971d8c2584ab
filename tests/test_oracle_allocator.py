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
    live = [b for s in pool.seqs.values() for b in s.table]
    assert sum(pool.refcount) == len(live)
    counts = np.bincount(np.asarray(live, dtype=np.int64), minlength=pool.num_blocks) if live else \
        np.zeros(pool.num_blocks, np.int64)
    assert list(counts) == pool.refcount
    free = pool.free_list()
    assert len(set(free)) == len(free)
    assert all(pool.refcount[b] == 0 for b in free)
    used = sum(1 for r in pool.refcount if r > 0)
    assert len(free) + used == pool.num_blocks
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
