"""The C-ABI library loads without a GPU, exports every function pkv.h declares,
and its host pool matches the oracle's pool model bit for bit (slots, copy pairs,
tables, refcounts, free-queue order, counters)."""

import ctypes

import numpy as np
import pytest

import paged_kv_cache_physical_amd as pk
import workloads as wl
from oracle import allocator as al
from oracle import run as orun
from paged_kv_cache_physical_amd import _lib


def test_exports_every_declared_symbol(libpkv):
    syms = _lib.header_symbols()
    assert len(syms) >= 18
    missing = [s for s in syms if not hasattr(libpkv, s)]
    assert missing == []
    assert pk.pkv_abi_version() == 11
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert libpkv.pkv_status_string(code) != b"unknown status"
    assert libpkv.pkv_status_string(-9) == b"unknown status"


def same_state(cpool: pk.Pool, opool: al.BlockPool):
    assert list(cpool.free_list()) == opool.free_list()
    assert [cpool.refcount(b) for b in range(opool.num_blocks)] == opool.refcount
    assert list(cpool.host_free_list()) == opool.host_free_list()
    assert [cpool.host_refcount(b) for b in range(opool.host_blocks)] == opool.host_refcount
    st = cpool.stats()
    assert st == {**opool.stats()}
    assert cpool.cached() == opool.cached
    for sid, s in opool.seqs.items():
        n, nb = cpool.info(sid)
        assert (n, nb) == (s.length, len(s.table))
        assert list(cpool.table(sid)) == s.table and cpool.on_host(sid) == s.on_host
    ids = sorted(sid for sid, s in opool.seqs.items() if not s.on_host)
    if ids:
        mb = max(1, max(len(opool.seqs[i].table) for i in ids))
        ct, cl = cpool.block_tables(ids, mb)
        ot, ol = opool.block_tables(ids, mb)
        assert np.array_equal(ct, ot) and np.array_equal(cl, ol)
    cpool.validate()


def test_worked_example(libpkv):
    for B, blocks in ((16, 62), (32, 32)):
        c = pk.Pool(128, B)
        ids = [c.create() for _ in range(5)]
        c.append(ids, [37, 91, 128, 201, 511])
        st = c.stats()
        assert st["logical_tokens"] == 968 and st["used_blocks"] == blocks and st["allocated_slots"] == blocks * B


def sharing_group(opool: al.BlockPool, sid: int):
    """sid and every sequence linked to it by a common block in the same tier."""
    group, todo = {sid}, [sid]
    while todo:
        s = opool.seqs[todo.pop()]
        for o, t in opool.seqs.items():
            if o not in group and t.on_host == s.on_host and set(t.table) & set(s.table):
                group.add(o)
                todo.append(o)
    return sorted(group)


def test_random_operations_match_oracle(libpkv):
    rng = np.random.default_rng(2024)
    errors = {al.OutOfBlocks: pk.OutOfBlocks, al.InvalidArg: pk.InvalidArg, al.WrongTier: pk.WrongTier}
    outcomes = {}
    for trial in range(30):
        nb = int(rng.integers(4, 60))
        B = int(rng.choice([1, 2, 4, 16, 32]))
        hb = int(rng.integers(0, 40))
        order = rng.permutation(nb)
        c, o = pk.Pool(nb, B, order, host_blocks=hb), al.BlockPool(nb, B, order, host_blocks=hb)
        live = []
        for _ in range(80):
            op = int(rng.integers(0, 8))
            if op == 0 or not live:
                a, b = c.create(), o.create()
                assert a == b
                live.append(a)
            elif op == 1:
                p = int(rng.choice(live))
                if o.on_host(p):
                    with pytest.raises(pk.WrongTier):
                        c.fork(p)
                    continue
                a, b = c.fork(p), o.fork(p)
                assert a == b
                live.append(a)
            elif op == 2:
                sid = int(rng.choice(live))
                c.free_seq(sid)
                o.free_seq(sid)
                live.remove(sid)
            elif op <= 4:
                k = int(rng.integers(1, len(live) + 1))
                seqs = [int(x) for x in rng.choice(live, size=k, replace=False)]
                counts = [int(x) for x in rng.integers(0, 3 * B + 2, size=k)]
                try:
                    so, po = o.append(seqs, counts)
                except (al.OutOfBlocks, al.WrongTier) as e:
                    with pytest.raises(errors[type(e)]):
                        c.append(seqs, counts)
                else:
                    sc, pc = c.append(seqs, counts)
                    assert np.array_equal(sc, so)
                    assert np.array_equal(pc, po)
            else:
                # swap a whole sharing group out or in; sometimes only part of it, or the wrong tier
                sid = int(rng.choice(live))
                group = sharing_group(o, sid)
                if op == 7 and len(group) > 1:
                    group = group[:-1]
                out = not o.on_host(sid) if op != 6 else o.on_host(sid)
                try:
                    po = o.swap_out(group) if out else o.swap_in(group)
                except (al.OutOfBlocks, al.InvalidArg, al.WrongTier) as e:
                    outcomes[type(e).__name__] = outcomes.get(type(e).__name__, 0) + 1
                    with pytest.raises(errors[type(e)]):
                        c.swap_out(group) if out else c.swap_in(group)
                else:
                    outcomes["out" if out else "in"] = outcomes.get("out" if out else "in", 0) + 1
                    pc = c.swap_out(group) if out else c.swap_in(group)
                    assert np.array_equal(pc, po)
            same_state(c, o)
    # every path was taken: swaps both ways and each refusal
    assert all(outcomes.get(k, 0) >= 5 for k in ("out", "in", "OutOfBlocks", "InvalidArg", "WrongTier")), outcomes


@pytest.mark.parametrize("name", ["tiny_f32", "llama7b_bf16", "gqa_bf16_b16", "gqa_bf16_b32", "beam_cow_bf16",
                                  "long_bf16"])
def test_workload_scripts_match_oracle(libpkv, name):
    w = wl.named(name, seed=0)
    rp = orun.replay(w, with_cache=False)
    c = pk.Pool(w.num_blocks, w.spec.block_size, w.free_order)
    k = 0
    for op in w.script():
        if isinstance(op, wl.Create):
            for _ in range(op.count):
                c.create()
        elif isinstance(op, wl.Fork):
            c.fork(op.parent)
        else:
            slots, pairs = c.append(op.seqs, op.counts)
            assert np.array_equal(slots, rp.slots[k]) and np.array_equal(pairs, rp.pairs[k])
            k += 1
    same_state(c, rp.pool)


def test_errors_leave_pool_unchanged(libpkv):
    c = pk.Pool(5, 4)
    a, b = c.create(), c.create()
    c.append([a, b], [6, 3])
    f = c.fork(a)
    before = (list(c.free_list()), [c.refcount(i) for i in range(5)], c.block_tables([a, b, f], 4))
    with pytest.raises(pk.OutOfBlocks):
        c.append([f, b, a], [3, 2, 3])
    with pytest.raises(pk.InvalidArg):
        c.append([a, a], [1, 1])
    with pytest.raises(pk.InvalidArg):
        c.append([a], [-1])
    with pytest.raises(pk.NoSuchSeq):
        c.append([a, 99], [1, 1])
    with pytest.raises(pk.NoSuchSeq):
        c.free_seq(99)
    with pytest.raises(pk.NoSuchSeq):
        c.fork(99)
    with pytest.raises(pk.InvalidArg):
        c.block_tables([a], 1)
    after = (list(c.free_list()), [c.refcount(i) for i in range(5)], c.block_tables([a, b, f], 4))
    assert before[0] == after[0] and before[1] == after[1]
    assert all(np.array_equal(x, y) for x, y in zip(before[2], after[2]))
    c.validate()
    c.free_seq(a)
    with pytest.raises(pk.NoSuchSeq):
        c.free_seq(a)  # double free
    assert c.refcount(-1) == -1 and c.refcount(5) == -1


def test_swap_errors_leave_pool_unchanged(libpkv):
    c = pk.Pool(6, 4, host_blocks=4)
    a = c.create()
    c.append([a], [6])
    b = c.fork(a)
    c.append([b], [1])
    x = c.create()
    c.append([x], [4])
    snap = lambda: (list(c.free_list()), list(c.host_free_list()), [c.refcount(i) for i in range(6)],
                    [c.host_refcount(i) for i in range(4)], [list(c.table(s)) for s in (a, b, x)])
    before = snap()
    with pytest.raises(pk.InvalidArg):
        c.swap_out([a])  # block 0 is also b's
    with pytest.raises(pk.InvalidArg):
        c.swap_out([a, a])
    with pytest.raises(pk.NoSuchSeq):
        c.swap_out([a, 42])
    with pytest.raises(pk.WrongTier):
        c.swap_in([a, b])
    c2 = pk.Pool(6, 4, host_blocks=2)
    y = c2.create()
    c2.append([y], [9])
    with pytest.raises(pk.OutOfBlocks):
        c2.swap_out([y])
    assert snap() == before
    c.swap_out([x])
    for call in (lambda: c.append([x], [1]), lambda: c.fork(x), lambda: c.block_tables([x], 4),
                 lambda: c.swap_out([x])):
        with pytest.raises(pk.WrongTier):
            call()
    with pytest.raises(pk.InvalidArg):
        pk.pkv_pool_set_host_blocks(c.handle, 8)  # a sequence is swapped out
    c.swap_in([x])
    pk.pkv_pool_set_host_blocks(c.handle, 8)
    assert c.stats()["host_blocks"] == 8 and list(c.host_free_list()) == list(range(8))
    c.validate()


def test_swap_pairs_capacity_reports_need(libpkv):
    L = libpkv
    c = pk.Pool(8, 4, host_blocks=8)
    s = c.create()
    c.append([s], [12])  # 3 blocks
    seqs = np.array([s], np.int32)
    n = ctypes.c_int32()
    st = L.pkv_swap_out(c.handle, seqs.ctypes.data_as(ctypes.c_void_p), 1, None, 0, ctypes.byref(n))
    assert st == _lib.PKV_ERR_INVALID_ARG and n.value == 3
    assert not c.on_host(s)
    c.validate()


def test_pool_create_rejects_bad_orders(libpkv):
    with pytest.raises(pk.InvalidArg):
        pk.Pool(3, 4, [0, 0, 1])
    with pytest.raises(pk.InvalidArg):
        pk.Pool(3, 4, [0, 1, 3])
    with pytest.raises(pk.InvalidArg):
        pk.Pool(0, 4)
    with pytest.raises(pk.InvalidArg):
        pk.Pool(4, 0)


def test_cow_capacity_error_reports_need(libpkv):
    L = libpkv
    c = pk.Pool(8, 4)
    p = c.create()
    c.append([p], [2])
    kids = [c.fork(p) for _ in range(2)]
    seqs = np.array(kids, np.int32)
    counts = np.ones(2, np.int32)
    slots = np.empty(2, np.int64)
    n = ctypes.c_int32()
    st = L.pkv_append_tokens(c.handle, seqs.ctypes.data_as(ctypes.c_void_p), counts.ctypes.data_as(ctypes.c_void_p),
                             2, None, slots.ctypes.data_as(ctypes.c_void_p), 2, None, 0, ctypes.byref(n))
    assert st == _lib.PKV_ERR_INVALID_ARG and n.value == 2
    c.validate()


def test_workspace_size_and_device_arg_checks(libpkv):
    # sizes are host arithmetic: 0 when one partition holds every sequence
    assert pk.pkv_attention_workspace_bytes(8, 32, 8, 128, 16, 32768, 0) == 0
    assert pk.pkv_attention_workspace_bytes(8, 32, 8, 128, 16, 512, 512) == 0
    assert pk.pkv_attention_workspace_bytes(8, 32, 6, 128, 16, 32768, 512) == 0  # 32 % 6 != 0
    # up to 4096 sequences: two records per workgroup of a grid of at most 2048
    # (here 8 x 8 heads x 64 partitions = 4096 items), each G x (d + 2) floats
    # plus a 16-byte header and a 16-byte hand-over pair
    nbytes = pk.pkv_attention_workspace_bytes(8, 32, 8, 128, 16, 32768, 512)
    recs = 2 * 2048
    assert recs * (4 * (128 + 2) * 4 + 32) <= nbytes <= recs * (4 * (128 + 2) * 4 + 32) + 5 * 256
    # few items: the grid, and so the records, shrink with them (2 x 8 heads x 2 partitions)
    small = pk.pkv_attention_workspace_bytes(2, 32, 8, 128, 16, 1024, 512)
    assert 2 * 32 * (4 * 130 * 4 + 32) <= small <= 2 * 32 * (4 * 130 * 4 + 32) + 5 * 256
    # above 4096 sequences: one slot per (sequence, query head, partition)
    big = pk.pkv_attention_workspace_bytes(5000, 8, 2, 64, 16, 1024, 512)
    rows = 5000 * 8 * 2
    assert rows * (64 + 3) * 4 <= big <= rows * (64 + 3) * 4 + 4 * 256
    # the static-scratch decode step refuses a batch whose workspace exceeds its 18 MiB before any device work
    # (5000 sequences take one slot per sequence, head and partition)
    assert libpkv.pkv_decode_step_static(None, None, None, None, None, None, None, None, 5000, 64, 8, 128, 16, 100000,
                                         128, 2048, ctypes.c_float(1.0), 16, 1, None) == _lib.PKV_ERR_WORKSPACE
    # argument errors are returned before anything touches a GPU
    L = libpkv
    vp = ctypes.c_void_p
    assert L.pkv_paged_attention_decode(None, None, None, None, None, None, 1, 6, 4, 128, 16, 10, 4, 64, 1.0, 0,
                                        None, 0, 1, None) == _lib.PKV_ERR_INVALID_ARG  # 6 % 4 != 0
    assert L.pkv_paged_attention_decode(None, None, None, None, None, None, 1, 48, 4, 128, 16, 10, 4, 64, 1.0, 0,
                                        None, 0, 1, None) == _lib.PKV_ERR_UNSUPPORTED  # G = 12
    assert L.pkv_paged_attention_decode(None, None, None, None, None, None, 1, 8, 8, 96, 16, 10, 4, 64, 1.0, 0,
                                        None, 0, 1, None) == _lib.PKV_ERR_UNSUPPORTED  # d = 96
    assert L.pkv_paged_attention_decode(None, None, None, None, None, None, 1, 8, 8, 128, 16, 10, 4, 64, 1.0, 24,
                                        None, 0, 1, None) == _lib.PKV_ERR_INVALID_ARG  # P % B != 0
    assert L.pkv_paged_attention_decode(None, None, None, None, None, None, 1, 8, 8, 128, 16, 10, 4, 64, 1.0, 0,
                                        None, 0, 7, None) == _lib.PKV_ERR_UNSUPPORTED  # dtype
    assert L.pkv_paged_attention_decode(None, None, None, None, None, None, 0, 8, 8, 128, 16, 10, 4, 64, 1.0, 0,
                                        None, 0, 1, None) == _lib.PKV_OK  # empty batch: no-op
    assert L.pkv_paged_attention_decode(None, None, None, None, None, None, 2, 8, 8, 128, 16, 10, 4, 64, 1.0, 0,
                                        None, 0, 1, None) == _lib.PKV_ERR_INVALID_ARG  # NULL buffers
    buf = [vp(4096)] * 6  # aligned stand-ins: every call below is rejected before any device work
    step_args = (2, 8, 8, 128, 16, 10, 4, 64, 1.0, 0, None, 0, 1, None)
    assert L.pkv_decode_step(None, None, *buf, *step_args) == _lib.PKV_ERR_INVALID_ARG  # no new token
    assert L.pkv_decode_step(vp(4096), None, *buf, *step_args) == _lib.PKV_ERR_INVALID_ARG  # K without V
    assert L.pkv_decode_step(vp(4104), vp(4096), *buf, *step_args) == _lib.PKV_ERR_INVALID_ARG  # misaligned K
    assert L.pkv_decode_step(vp(4096), vp(4096), None, *buf[1:], *step_args) == _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_reshape_and_cache(None, None, None, None, None, 0, 8, 128, 16, 10, 1, None) == _lib.PKV_OK
    assert L.pkv_reshape_and_cache(None, None, None, None, None, 3, 8, 128, 16, 10, 1, None) == _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_reshape_and_cache(None, None, None, None, None, 3, 8, 128, 24, 10, 1, None) == _lib.PKV_ERR_UNSUPPORTED
    assert L.pkv_copy_blocks(None, None, None, 0, 10, 4096, None) == _lib.PKV_OK
    assert L.pkv_copy_blocks(None, None, None, 2, 10, 4096, None) == _lib.PKV_ERR_INVALID_ARG
    assert L.pkv_copy_blocks(vp(16), vp(16), vp(16), 2, 10, 4100, None) == _lib.PKV_ERR_INVALID_ARG


def test_prefix_cache_by_hand_matches_oracle(libpkv):
    """The oracle's hand-traced prefix-cache scenario, replayed on both pools in lockstep."""
    c, o = pk.Pool(8, 4), al.BlockPool(8, 4)

    def both(fn):
        a, b = fn(c), fn(o)
        same_state(c, o)
        return a, b

    a, _ = both(lambda p: p.create())
    (sc, _), (so, _) = both(lambda p: p.append([a], [10], token_ids=list(range(1, 11))))
    assert np.array_equal(sc, so)
    k0 = al.block_key(0, [1, 2, 3, 4])
    assert c.cached() == {k0: 0, al.block_key(k0, [5, 6, 7, 8]): 1}  # FNV-1a chain in C equals the oracle's
    (b, hc), (_, ho) = both(lambda p: p.create_prefixed([1, 2, 3, 4, 5, 6, 7, 8, 11, 12]))
    assert hc == ho == 8
    both(lambda p: p.append([b], [2], token_ids=[11, 12]))
    (cc, hc), (_, ho) = both(lambda p: p.create_prefixed([1, 2, 3, 4, 5, 6, 7, 8]))
    assert hc == ho == 4
    both(lambda p: p.append([cc], [4], token_ids=[5, 6, 7, 8]))
    both(lambda p: p.free_seq(a))
    both(lambda p: p.free_seq(b))
    (d, _), _ = both(lambda p: p.create_prefixed([1, 2, 3, 4, 5, 6, 7, 8, 9]))
    e, _ = both(lambda p: p.create())
    both(lambda p: p.append([e], [16]))
    both(lambda p: p.free_seq(d))
    f, _ = both(lambda p: p.create())
    both(lambda p: p.append([f], [8]))
    (_, hc), (_, ho) = both(lambda p: p.create_prefixed([1, 2, 3, 4, 5, 6, 7, 8, 9]))
    assert hc == ho == 4
    c.validate()


def test_prefix_cache_random_operations_match_oracle(libpkv):
    """Random prompts from a few shared stems, appends with and without ids, forks, frees and swaps: the C pool
    and the oracle agree on every slot, copy pair, hit length, table, queue and key after every step."""
    rng = np.random.default_rng(91)
    hits = 0
    for trial in range(25):
        B = int(rng.choice([1, 2, 4, 16]))
        nb, hb = int(rng.integers(8, 60)), int(rng.integers(0, 30))
        order = rng.permutation(nb)
        c, o = pk.Pool(nb, B, order, host_blocks=hb), al.BlockPool(nb, B, order, host_blocks=hb)
        stems = [[int(x) for x in rng.integers(0, 3, size=int(rng.integers(1, 3 * B + 3)))] for _ in range(4)]
        for _ in range(70):
            op = int(rng.integers(0, 7))
            dev = [s for s in o.seqs if not o.on_host(s)]
            if op == 0 or not dev:
                ids = stems[int(rng.integers(0, 4))] + [int(x) for x in rng.integers(0, 3, size=int(rng.integers(0, 6)))]
                sc, hc = c.create_prefixed(ids)
                so, ho = o.create_prefixed(ids)
                assert (sc, hc) == (so, ho)
                hits += hc // B
                try:
                    res_o = o.append([so], [len(ids) - ho], token_ids=ids[ho:])
                except al.OutOfBlocks:
                    with pytest.raises(pk.OutOfBlocks):
                        c.append([sc], [len(ids) - hc], token_ids=ids[hc:])
                    c.free_seq(sc)
                    o.free_seq(so)
                else:
                    res_c = c.append([sc], [len(ids) - hc], token_ids=ids[hc:])
                    assert all(np.array_equal(x, y) for x, y in zip(res_c, res_o))
            elif op == 1:
                sid = int(rng.choice(list(o.seqs)))
                c.free_seq(sid)
                o.free_seq(sid)
            elif op in (2, 3):
                k = int(rng.integers(1, len(dev) + 1))
                seqs = [int(x) for x in rng.choice(dev, size=k, replace=False)]
                counts = [int(x) for x in rng.integers(0, 2 * B + 2, size=k)]
                ids = None if op == 3 and rng.random() < 0.4 else [int(x) for x in rng.integers(0, 3, size=sum(counts))]
                try:
                    res_o = o.append(seqs, counts, token_ids=ids)
                except al.OutOfBlocks:
                    with pytest.raises(pk.OutOfBlocks):
                        c.append(seqs, counts, token_ids=ids)
                else:
                    res_c = c.append(seqs, counts, token_ids=ids)
                    assert all(np.array_equal(x, y) for x, y in zip(res_c, res_o))
            elif op == 4:
                p = int(rng.choice(dev))
                assert c.fork(p) == o.fork(p)
            else:
                sid = int(rng.choice(list(o.seqs)))
                group = sharing_group(o, sid)
                out = not o.on_host(sid)
                try:
                    po = o.swap_out(group) if out else o.swap_in(group)
                except (al.OutOfBlocks, al.InvalidArg) as e:
                    with pytest.raises({al.OutOfBlocks: pk.OutOfBlocks, al.InvalidArg: pk.InvalidArg}[type(e)]):
                        c.swap_out(group) if out else c.swap_in(group)
                else:
                    pc = c.swap_out(group) if out else c.swap_in(group)
                    assert np.array_equal(pc, po)
            same_state(c, o)
    assert hits > 100  # the stems make the cache hit often


def test_prefix_cache_argument_errors(libpkv):
    c = pk.Pool(8, 4)
    with pytest.raises(pk.InvalidArg):
        c.append([c.create()], [3], token_ids=[1, 2])  # one id per token
    sid, hit = c.create_prefixed([])
    assert hit == 0 and c.info(sid) == (0, 0)
    n_seq, hit = ctypes.c_int32(), ctypes.c_int32()
    assert libpkv.pkv_seq_create_prefixed(c.handle, None, 3, ctypes.byref(n_seq), ctypes.byref(hit)) == \
        _lib.PKV_ERR_INVALID_ARG
    assert libpkv.pkv_seq_create_prefixed(c.handle, None, -1, ctypes.byref(n_seq), ctypes.byref(hit)) == \
        _lib.PKV_ERR_INVALID_ARG
    n = ctypes.c_int32()
    c.append([sid], [4], token_ids=[1, 2, 3, 4])
    assert libpkv.pkv_pool_cached_blocks(c.handle, None, None, 0, ctypes.byref(n)) == _lib.PKV_ERR_INVALID_ARG
    assert n.value == 1
    c.validate()


def test_truncate_matches_oracle(libpkv):
    """The oracle's hand-traced rollbacks and random operations with truncation, on both pools in lockstep."""
    for B, script in ((4, "hand"), (4, "keys")):
        c, o = pk.Pool(8 if script == "hand" else 6, B), al.BlockPool(8 if script == "hand" else 6, B)
        if script == "hand":
            a = c.create(); o.create()
            c.append([a], [10]); o.append([a], [10])
            b = c.fork(a); o.fork(a)
            c.truncate(b, 5); o.truncate(b, 5)
            same_state(c, o)
            (sc, pc), (so, po) = c.append([b], [1]), o.append([b], [1])
            assert np.array_equal(sc, so) and np.array_equal(pc, po) and pc.tolist() == [[1, 3]]
            c.truncate(a, 0); o.truncate(a, 0)
            same_state(c, o)
            c.truncate(b, 4); o.truncate(b, 4)
            for bad in (5, -1):
                with pytest.raises(pk.InvalidArg):
                    c.truncate(b, bad)
        else:
            a = c.create(); o.create()
            ids = [1, 2, 3, 4, 5, 6, 7, 8]
            c.append([a], [8], token_ids=ids); o.append([a], [8], token_ids=ids)
            c.truncate(a, 6); o.truncate(a, 6)
            assert c.create_prefixed(ids + [9]) == o.create_prefixed(ids + [9])
            c.append([a], [1]); o.append([a], [1])
            x = c.create(); o.create()
            c.append([x], [8], token_ids=[9, 9, 9, 9, 8, 8, 8, 8]); o.append([x], [8], token_ids=[9, 9, 9, 9, 8, 8, 8, 8])
            c.truncate(x, 5); o.truncate(x, 5)
            c.append([x], [1]); o.append([x], [1])
            c.append([x], [2], token_ids=[8, 8]); o.append([x], [2], token_ids=[8, 8])
        same_state(c, o)
        c.validate()
    rng = np.random.default_rng(33)
    for trial in range(20):
        B = int(rng.choice([1, 2, 4, 16]))
        nb, hb = int(rng.integers(8, 50)), int(rng.integers(0, 20))
        order = rng.permutation(nb)
        c, o = pk.Pool(nb, B, order, host_blocks=hb), al.BlockPool(nb, B, order, host_blocks=hb)
        stem = [int(x) for x in rng.integers(0, 2, size=2 * B + 1)]
        for _ in range(80):
            op = int(rng.integers(0, 7))
            dev = [s for s in o.seqs if not o.on_host(s)]
            if op == 0 or not dev:
                ids = stem + [int(x) for x in rng.integers(0, 2, size=int(rng.integers(0, 4)))]
                assert c.create_prefixed(ids) == o.create_prefixed(ids)
            elif op == 1:
                sid = int(rng.choice(dev))
                n = int(rng.integers(1, 2 * B + 2))
                ids = [int(x) for x in rng.integers(0, 2, size=n)] if rng.random() < 0.8 else None
                try:
                    res_o = o.append([sid], [n], token_ids=ids)
                except al.OutOfBlocks:
                    with pytest.raises(pk.OutOfBlocks):
                        c.append([sid], [n], token_ids=ids)
                else:
                    res_c = c.append([sid], [n], token_ids=ids)
                    assert all(np.array_equal(x, y) for x, y in zip(res_c, res_o))
            elif op == 2:
                p = int(rng.choice(dev))
                assert c.fork(p) == o.fork(p)
            elif op in (3, 4):
                sid = int(rng.choice(list(o.seqs)))
                if o.on_host(sid):
                    with pytest.raises(pk.WrongTier):
                        c.truncate(sid, 0)
                    continue
                n = int(rng.integers(0, o.length(sid) + 1))
                c.truncate(sid, n)
                o.truncate(sid, n)
            elif op == 5:
                sid = int(rng.choice(list(o.seqs)))
                c.free_seq(sid)
                o.free_seq(sid)
            else:
                sid = int(rng.choice(list(o.seqs)))
                group = sharing_group(o, sid)
                out = not o.on_host(sid)
                try:
                    po = o.swap_out(group) if out else o.swap_in(group)
                except (al.OutOfBlocks, al.InvalidArg) as e:
                    with pytest.raises({al.OutOfBlocks: pk.OutOfBlocks, al.InvalidArg: pk.InvalidArg}[type(e)]):
                        c.swap_out(group) if out else c.swap_in(group)
                else:
                    assert np.array_equal(c.swap_out(group) if out else c.swap_in(group), po)
            same_state(c, o)


def test_duplicate_and_unknown_ids_in_one_append(libpkv):
    """A sequence listed twice is an argument error before any unknown id is reported, whether or not the
    id exists, on both pools."""
    c, o = pk.Pool(8, 4), al.BlockPool(8, 4)
    c.create(), o.create()
    for seqs, err in (([99, 99], pk.InvalidArg), ([-3, -3], pk.InvalidArg), ([0, 0], pk.InvalidArg),
                      ([99, -3], pk.NoSuchSeq), ([0, 7, 0], pk.InvalidArg)):
        with pytest.raises({pk.InvalidArg: al.InvalidArg, pk.NoSuchSeq: al.NoSuchSeq}[err]):
            o.append(seqs, [1] * len(seqs))
        with pytest.raises(err):
            c.append(seqs, [1] * len(seqs))
        same_state(c, o)
    # many calls in a row keep their duplicate checks separate
    for _ in range(5):
        c.append([0], [1])
        o.append([0], [1])
    same_state(c, o)


def listed_runs_bytes(S, Hq, Hkv, d, ctx, mq):
    """The decode kernel's path for runs of at most 16 / G queries (all the runs when mq * G <= 16, else the short
    runs of a mixed batch): records of 16 columns for two per workgroup of a grid of at most 2048 (a multiple of
    H_kv), over 512-token partitions (256 when the batch's groups at its longest context stay under six 40-unit
    partitions per lane of 512 / H_kv workgroups); 0 when no context is cut."""
    lanes = max(1, 512 // Hkv)
    P = 256 if S * (-(-ctx // 16)) < 6 * lanes * 40 else 512
    parts = -(-max(ctx, 1) // P)
    if parts <= 1:
        return 0
    items = parts * S * Hkv
    grid = min(items, 2048) // Hkv * Hkv
    up = lambda x: (x + 255) // 256 * 256
    recs = 2 * grid
    return up(recs * 16 * d * 4) + 2 * up(recs * 16 * 4) + up(recs * 16) + up(recs * 16)


def test_runs_of_queries_host_checks_and_split_plan(libpkv):
    """pkv_paged_attention_multi rejects bad arguments before any device work, and the workspace is the larger of
    the two paths' needs: the runs kernel's split plan (>= 256-token splits for about 2048 workgroups, at most 64,
    only when a pair's rows fit 64) and the decode kernel's records for short runs (16 / G queries at most)."""
    L = libpkv
    vp = ctypes.c_void_p
    # (num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, max_query_len) -> bytes
    assert pk.pkv_attention_multi_workspace_bytes(8, 32, 8, 128, 32768, 4) == max(
        64 * 32 * 64 * 130 * 4, listed_runs_bytes(8, 32, 8, 128, 32768, 4))
    assert pk.pkv_attention_multi_workspace_bytes(3, 8, 2, 64, 600, 5) == 6 * 2 * 64 * 66 * 4  # 20 columns
    assert listed_runs_bytes(1, 8, 8, 128, 1 << 20, 1) > 8 * 64 * 64 * 130 * 4
    assert pk.pkv_attention_multi_workspace_bytes(1, 8, 8, 128, 1 << 20, 1) == listed_runs_bytes(
        1, 8, 8, 128, 1 << 20, 1)  # the runs kernel's split is capped at 64
    # enough pairs for the runs kernel; the short runs still cut their 2048-token contexts
    assert pk.pkv_attention_multi_workspace_bytes(64, 32, 32, 128, 2048, 4) == listed_runs_bytes(
        64, 32, 32, 128, 2048, 4) > 0
    # 68 rows: the runs kernel does not split, but the short runs of such a batch take the decode kernel's path
    assert pk.pkv_attention_multi_workspace_bytes(8, 32, 8, 128, 32768, 17) == listed_runs_bytes(
        8, 32, 8, 128, 32768, 17) > 0
    # a small batch's short runs take 256-token partitions: 500-token contexts are cut, 256-token ones are not
    assert pk.pkv_attention_multi_workspace_bytes(8, 32, 8, 128, 500, 4) == listed_runs_bytes(
        8, 32, 8, 128, 500, 4) > 0
    assert pk.pkv_attention_multi_workspace_bytes(8, 32, 8, 128, 256, 4) == 0  # too short to split
    assert pk.pkv_attention_multi_workspace_bytes(8, 30, 8, 128, 32768, 4) == 0  # H_q % H_kv != 0

    def call(out=None, q=None, k=None, v=None, bt=None, cl=None, qs=None, order=None, S=2, T=8, Hq=8, Hkv=8, d=128,
             B=16, nb=10, mb=4, mctx=64, mq=4, scale=1.0, ws=None, wsb=0, dt=1):
        return L.pkv_paged_attention_multi(out, q, k, v, bt, cl, qs, order, S, T, Hq, Hkv, d, B, nb, mb, mctx, mq,
                                           scale, ws, wsb, dt, None)
    assert call(dt=7) == _lib.PKV_ERR_UNSUPPORTED
    assert call(Hq=6, Hkv=4) == _lib.PKV_ERR_INVALID_ARG
    assert call(Hq=48, Hkv=4) == _lib.PKV_ERR_UNSUPPORTED  # G = 12
    assert call(d=96) == _lib.PKV_ERR_UNSUPPORTED
    assert call(B=24) == _lib.PKV_ERR_UNSUPPORTED
    assert call(scale=float("nan")) == _lib.PKV_ERR_INVALID_ARG
    assert call(mq=-1) == _lib.PKV_ERR_INVALID_ARG
    assert call(S=0) == _lib.PKV_OK and call(mq=0) == _lib.PKV_OK and call(T=0) == _lib.PKV_OK  # nothing to do
    assert call() == _lib.PKV_ERR_INVALID_ARG  # NULL buffers
    buf = [vp(4096)] * 7  # aligned stand-ins: every call below is rejected before any device work
    assert call(*buf[:2], vp(4104), *buf[3:]) == _lib.PKV_ERR_INVALID_ARG  # misaligned key cache
    need = pk.pkv_attention_multi_workspace_bytes(8, 32, 8, 128, 32768, 4)
    split = dict(S=8, Hq=32, Hkv=8, mctx=32768, mb=2048, nb=16384)
    assert call(*buf, **split, ws=vp(4096), wsb=need - 1) == _lib.PKV_ERR_WORKSPACE
    assert call(*buf, **split, ws=vp(4104), wsb=need) == _lib.PKV_ERR_WORKSPACE  # misaligned workspace


def test_freed_blocks_wait_out_every_earlier_free_block(libpkv):
    """The C pool hands a freed block out again only after every block that was free before it (FIFO)."""
    c = pk.Pool(12, 4)
    a, b = c.create(), c.create()
    c.append([a], [16])  # blocks 0-3
    c.append([b], [8])   # blocks 4-5
    c.free_seq(a)        # 0-3 join the tail, behind 6-11
    assert list(c.free_list()) == [6, 7, 8, 9, 10, 11, 0, 1, 2, 3]
    x = c.create()
    slots, _ = c.append([x], [24])  # six blocks: every never-used one first
    assert sorted(set((slots // 4).tolist())) == [6, 7, 8, 9, 10, 11]
    y = c.create()
    slots, _ = c.append([y], [5])
    assert (slots // 4).tolist() == [0, 0, 0, 0, 1]  # then the oldest freed, in release order
