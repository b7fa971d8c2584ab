"""GPU parity: the HIP path (through the C-ABI) against the float64 oracle.

Bars: block tables, slots and cache bytes bit-exact; fp32 caches max abs error
<= 1e-5; bf16 caches max abs <= 1e-2 and relative L2 <= 2e-3.  Because a single
dropped token can hide under the bf16 bar, every case also meets a tighter
bound derived from fp32 accumulation (relative L2 <= 1e-4).
"""

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oa
from oracle import cache as oc
from oracle import run as orun

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu(libpkv):
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    yield
    torch.cuda.synchronize()


def runner():
    from paged_kv_cache_physical_amd.runner import GpuBatch
    return GpuBatch


def say(*a):
    print(*a, flush=True)


def host_bits(t):
    """Device cache tensor -> host NumPy array with the oracle's storage dtype."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def same_bits(a, b):
    """Bit-for-bit equality (NaN poison included)."""
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and a.dtype == b.dtype and a.tobytes() == b.tobytes()


def check_close(out, ref, kv_dtype, what=""):
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = float(np.max(np.abs(out - ref)))
    rl2 = float(np.linalg.norm(out - ref) / np.linalg.norm(ref))
    say(f"  {what}: max_abs={err:.3e} rel_l2={rl2:.3e}")
    if kv_dtype == "f32":
        assert err <= 1e-5, (what, err)
    else:
        assert err <= 1e-2 and rl2 <= 2e-3, (what, err, rl2)
    assert rl2 <= 1e-4, (what, rl2)


def full_parity(w, partitions):
    GpuBatch = runner()
    s = w.spec
    say(f"case {s.name}: S={w.num_seqs} Hq={s.num_q_heads} Hkv={s.num_kv_heads} d={s.head_dim} B={s.block_size} "
        f"{s.kv_dtype} max_n={w.max_context_len}")
    gb = GpuBatch(w)
    rp = orun.replay(w)
    assert np.array_equal(gb.tables_host[:, :rp.tables.shape[1]], rp.tables)
    assert np.all(gb.tables_host[:, rp.tables.shape[1]:] == -1)
    assert np.array_equal(gb.lens_host, rp.context_lens)
    for a, b in zip(gb.slots, rp.slots):
        assert np.array_equal(a, b)
    assert same_bits(host_bits(gb.k_cache), rp.k_cache)
    assert same_bits(host_bits(gb.v_cache), rp.v_cache)
    ref = oa.paged_attention(w.q, rp.k_cache, rp.v_cache, rp.tables, rp.context_lens, w.scale, s.kv_dtype)
    outs = {}
    for P in partitions:
        out = gb.attention(P).cpu().numpy()
        torch.cuda.synchronize()
        check_close(out, ref, s.kv_dtype, f"P={P}")
        outs[P] = out
    return gb, outs


@pytest.mark.parametrize("P", [0, 16, 64, 512])
def test_tiny_f32(P):
    full_parity(wl.named("tiny_f32", seed=0), [P])


GRID = [(dt, d, G, B) for dt in ("f32", "bf16") for d in (64, 128) for G in (1, 2, 4, 8) for B in (16, 32)]


@pytest.mark.parametrize("dt,d,G,B", GRID)
def test_small_grid(dt, d, G, B):
    w = wl.small_decode(7, (1, 300), 2 * G, 2, d, B, dt, seed=G * 100 + d + B)
    full_parity(w, [0, 2 * B, 160 if B == 16 else 192])


@pytest.mark.parametrize("G,lens", [(8, (513, 2000)), (4, (1025, 1500)), (1, (4097, 5000)), (2, (1, 2100))])
def test_multi_chunk_unsplit(G, lens):
    # one partition longer than a chunk (4096 / G tokens): the chunked online-softmax kernel
    w = wl.small_decode(3, lens, 2 * G, 2, 128, 16, "bf16", seed=7 + G)
    full_parity(w, [0, 4096 // G + 16 * 3])


@pytest.mark.parametrize("case", range(16))
def test_random_batches_match_oracle(case):
    # seeded random batches: every (dtype, d, G) pair, random block size, KV
    # head count, batch size, lengths and partition sizes, so each kernel
    # instantiation sees runs cut at many places and ragged tails
    rng = np.random.default_rng(1000 + case)
    dt = ("f32", "bf16")[case % 2]
    d = (64, 128)[(case // 2) % 2]
    G = (1, 2, 4, 8)[(case // 4) % 4]
    B = (16, 32)[int(rng.integers(2))]
    Hkv = int(rng.choice([1, 2, 4]))
    S = int(rng.integers(20, 200))
    hi = int(rng.integers(64, 3000))
    w = wl.small_decode(S, (1, hi), G * Hkv, Hkv, d, B, dt, seed=case)
    parts = sorted({0, B * int(rng.integers(1, 9)), B * int(rng.integers(8, 40))})
    full_parity(w, parts)


def test_ragged_boundaries():
    # lengths at block, partition and chunk edges
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025]
    w = wl.small_decode(len(lens), (1, 1), 16, 2, 128, 16, "bf16", seed=3, lens=lens)
    full_parity(w, [0, 64, 512])


@pytest.mark.parametrize("dt,d,G,B", [("bf16", 128, 1, 16), ("bf16", 128, 8, 32), ("bf16", 64, 4, 16),
                                       ("f32", 128, 2, 32)])
def test_many_items_per_workgroup(dt, d, G, B):
    # more items than the persistent grid holds: each workgroup walks several
    # items, many shorter than one turn of its load ring, so the ring's
    # look-ahead crosses item boundaries (into items of every length)
    w = wl.small_decode(600, (1, 200), 2 * G, 2, d, B, dt, seed=11 + G + d + B)
    full_parity(w, [0, 2 * B])


def test_more_sequences_than_the_item_list_holds():
    # above 4096 sequences the items are numbered without the LDS list and the
    # empty ones are skipped
    w = wl.small_decode(4200, (1, 40), 2, 1, 64, 16, "bf16", seed=21)
    full_parity(w, [0, 16])


@pytest.mark.parametrize("name", ["llama7b_bf16", "gqa_bf16_b16", "gqa_bf16_b32", "beam_cow_bf16", "long_bf16"])
def test_named_full_size(name):
    """A full-size workload, every output row against the float64 oracle (the contiguous-KV baseline of the
    guide's verification protocol): block tables and lengths equal the oracle pool's, both whole caches equal the
    oracle's own scatter bit for bit (unwritten slots' NaN poison included), and the attention output over all
    S x H_q x d elements meets the bars at the workload's partition size and unsplit, as does the decode step
    (token write plus attention), which is also idempotent."""
    GpuBatch = runner()
    w = wl.named(name, seed=0)
    s = w.spec
    say(f"case {name}: S={w.num_seqs} tokens={w.total_tokens} pool={w.num_blocks}")
    gb = GpuBatch(w)
    rp = orun.replay(w)
    assert np.array_equal(gb.tables_host[:, :rp.tables.shape[1]], rp.tables)
    assert np.all(gb.tables_host[:, rp.tables.shape[1]:] == -1)
    assert np.array_equal(gb.lens_host, rp.context_lens)
    assert same_bits(host_bits(gb.k_cache), rp.k_cache), "key cache bytes"
    assert same_bits(host_bits(gb.v_cache), rp.v_cache), "value cache bytes"
    ref = oa.paged_attention(w.q, rp.k_cache, rp.v_cache, rp.tables, rp.context_lens, w.scale, s.kv_dtype)
    del rp
    say(f"  oracle: {ref.shape[0]} sequences x {ref.shape[1]} heads x {ref.shape[2]} dims")
    for P in sorted({s.partition_size, 0}):
        out = gb.attention(P).cpu().numpy()
        check_close(out, ref, s.kv_dtype, f"{name} P={P}, all rows")
    out1 = gb.step().cpu().numpy()
    check_close(out1, ref, s.kv_dtype, f"{name} decode step, all rows")
    out2 = gb.step().cpu().numpy()
    assert np.array_equal(out1, out2)


def test_placement_invariance_bitwise():
    GpuBatch = runner()
    w1 = wl.small_decode(9, (1, 700), 16, 2, 128, 16, "bf16", seed=5)
    w2 = wl.small_decode(9, (1, 700), 16, 2, 128, 16, "bf16", seed=5)
    w2.free_order = np.random.default_rng(77).permutation(w2.num_blocks).astype(np.int32)
    g1, g2 = GpuBatch(w1), GpuBatch(w2)
    assert not np.array_equal(g1.tables_host, g2.tables_host)
    for P in (0, 64):
        a = g1.attention(P).cpu().numpy()
        b = g2.attention(P).cpu().numpy()
        assert np.array_equal(a, b), P


def test_shared_prefix_equals_private_bitwise():
    import paged_kv_cache_physical_amd as pk
    GpuBatch = runner()
    w = wl.named("beam_cow_bf16", seed=2, prompts=4, prefix_len=200, tail_range=(1, 40), num_blocks=256)
    s = w.spec
    shared = GpuBatch(w)
    rp = orun.replay(w)
    # copy-on-write and writes: the whole pool matches the oracle's bytes
    assert same_bits(host_bits(shared.k_cache), rp.k_cache)
    assert same_bits(host_bits(shared.v_cache), rp.v_cache)
    assert sum(len(p) for p in shared.pairs) == s.prompts * (s.beams - 1)
    # private copies of every beam in a second pool
    pool = pk.Pool(w.num_blocks * 2, s.block_size)
    kc, vc = pk.empty_caches(w.num_blocks * 2, s.num_kv_heads, s.block_size, s.head_dim, "bf16")
    from paged_kv_cache_physical_amd.runner import _to_device
    ids = []
    for i in range(w.num_seqs):
        sid = pool.create()
        ids.append(sid)
        slots, _ = pool.append([sid], [int(w.context_lens[i])])
        k, v = w.token_kv(i)
        pk.pkv_reshape_and_cache(_to_device(k, "bf16", "cuda"), _to_device(v, "bf16", "cuda"), kc, vc,
                                 torch.from_numpy(slots).cuda(), s.block_size)
    mb = shared.max_blocks
    tables, lens = pool.block_tables(ids, mb)
    out_p = torch.empty_like(shared.out)
    for P in (0, 64):
        pk.pkv_paged_attention_decode(out_p, shared.q, kc, vc, torch.from_numpy(tables).cuda(),
                                      torch.from_numpy(lens).cuda(), shared.max_context_len, float(w.scale), P,
                                      shared.workspace(P))
        a = shared.attention(P).cpu().numpy()
        assert np.array_equal(a, out_p.cpu().numpy()), P
        ref = oa.paged_attention(w.q, rp.k_cache, rp.v_cache, rp.tables, rp.context_lens, w.scale, "bf16")
        check_close(a, ref, "bf16", f"beam P={P}")


def test_split_matches_unsplit():
    GpuBatch = runner()
    w = wl.small_decode(6, (200, 1500), 32, 8, 128, 16, "bf16", seed=9)
    gb = GpuBatch(w)
    a = gb.attention(0).cpu().numpy()
    for P in (16, 48, 512):
        b = gb.attention(P).cpu().numpy()
        assert float(np.linalg.norm(a - b) / np.linalg.norm(a)) <= 1e-5


def test_fine_lane_cuts_match_oracle():
    # enough work per lane that runs are cut at group granularity: segments
    # start mid-partition (partition 0 included, which uses slot 1)
    w = wl.small_decode(300, (100, 2000), 8, 2, 128, 16, "bf16", seed=13)
    full_parity(w, [256, 512])


@pytest.mark.parametrize("nseq,lens,P", [(300, (100, 2000), 256), (6, (200, 1500), 48)])
def test_two_stage_equals_fused_with_stale_workspace(nseq, lens, P):
    # partitions then reduce (separate calls) give the fused call's bits, and
    # whatever the workspace held before does not leak into the result
    GpuBatch = runner()
    w = wl.small_decode(nseq, lens, 8, 2, 128, 16, "bf16", seed=17)
    gb = GpuBatch(w)
    fused = gb.attention(P).clone()
    ws = gb.workspace(P)
    assert ws is not None
    for fill in (0x00, 0x7F, 0xFF):
        ws.fill_(fill)
        gb.out.fill_(float("nan"))
        gb.attention_partitions(P)
        gb.attention_reduce(P)
        torch.cuda.synchronize()
        assert torch.equal(gb.out, fused), fill


@pytest.mark.parametrize("nseq,lens,P", [(300, (100, 2000), 256), (6, (200, 1500), 48), (8, (20000, 32768), 512)])
def test_fused_combine_needs_no_clean_workspace(nseq, lens, P):
    # The one-call path combines a cut sequence inside the kernel: the owner
    # waits for the earlier runs' records through (turn, flag) pairs in the
    # workspace.  Starting from zeros, 0xFF bytes, random bytes, consecutive
    # int64 values (equal neighbours off by one), and a workspace last used by
    # a batch of another shape, every call gives the two-stage path's bits,
    # on repeated calls too; the last case spans each sequence over dozens of
    # runs (long chains of records, empty runs inside them).
    import paged_kv_cache_physical_amd as pk
    GpuBatch = runner()
    w = wl.small_decode(nseq, lens, 8, 2, 128, 16, "bf16", seed=19)
    gb = GpuBatch(w)
    ws = gb.workspace(P)
    assert ws is not None
    gb.out.fill_(float("nan"))
    gb.attention_partitions(P)
    gb.attention_reduce(P)
    torch.cuda.synchronize()
    ref = gb.out.clone()
    assert bool(torch.isfinite(ref).all())
    gen = torch.Generator(device="cuda").manual_seed(5)
    fills = {"zeros": lambda: ws.zero_(), "0xff": lambda: ws.fill_(0xFF),
             "random": lambda: ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda",
                                                      generator=gen)),
             "count": lambda: ws.view(torch.int64).copy_(torch.arange(ws.numel() // 8, device="cuda"))}
    for name, fill in fills.items():
        fill()
        for rep in range(3):
            gb.out.fill_(float("nan"))
            gb.attention(P)
            torch.cuda.synchronize()
            assert torch.equal(gb.out, ref), (name, rep)
    # the same buffer for a batch of another shape (G = 4 over 8 KV heads, d = 64, B = 32), then back
    w2 = wl.small_decode(50, (10, 3000), 32, 8, 64, 32, "bf16", seed=20)
    g2 = GpuBatch(w2)
    P2 = 64
    need = pk.pkv_attention_workspace_bytes(w2.num_seqs, 32, 8, 64, 32, g2.max_context_len, P2)
    ws2 = ws if need <= ws.numel() else torch.zeros(need, dtype=torch.uint8, device="cuda")
    g2.attention_partitions(P2)
    g2.attention_reduce(P2)
    torch.cuda.synchronize()
    ref2 = g2.out.clone()
    for rep in range(2):
        g2.out.fill_(float("nan"))
        pk.pkv_paged_attention_decode(g2.out, g2.q, g2.k_cache, g2.v_cache, g2.block_tables, g2.context_lens,
                                      g2.max_context_len, float(w2.scale), P2, ws2)
        torch.cuda.synchronize()
        assert torch.equal(g2.out, ref2), rep
        gb.out.fill_(float("nan"))
        gb.attention(P)
        torch.cuda.synchronize()
        assert torch.equal(gb.out, ref), rep


@pytest.mark.parametrize("name", ["gqa_bf16_b16", "long_bf16"])
def test_repeated_calls_are_bitwise_stable(name):
    # the same inputs give the same bits on every call
    GpuBatch = runner()
    w = wl.named(name, seed=3)
    gb = GpuBatch(w)
    P = w.spec.partition_size
    first = gb.attention(P).clone()
    for i in range(12):
        gb.out.fill_(float("nan"))
        gb.attention(P)
        torch.cuda.synchronize()
        assert torch.equal(gb.out, first), i


def test_step_replays_as_a_graph():
    # the decode step (token write, partitions, reduction) captured as a HIP
    # graph gives the eager step's bits on every replay, with eager work and
    # synchronisations between the replays
    GpuBatch = runner()
    w = wl.small_decode(40, (100, 3000), 16, 4, 128, 16, "bf16", seed=23)
    gb = GpuBatch(w)
    P = 256
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = gb.step(P, stream=s).clone()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            gb.step(P, stream=s)
        for i in range(4):
            gb.out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(gb.out, eager), i
            gb.out.fill_(float("nan"))
            gb.attention(P, stream=s)
            torch.cuda.synchronize()
            assert torch.equal(gb.out, eager), i


def cache_bits(t):
    """Integer view of a device cache, so NaN poison compares bit for bit."""
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def poison_decode_slots(gb):
    """Overwrite every sequence's decode-token slot with NaN."""
    import paged_kv_cache_physical_amd as pk
    d = gb.decode
    pk.pkv_reshape_and_cache(torch.full_like(d.k_new, float("nan")), torch.full_like(d.v_new, float("nan")),
                             gb.k_cache, gb.v_cache, d.slots, gb.workload.spec.block_size)


DECODE_STEP_CASES = [
    # (seqs, lengths, G, H_kv, d, B, dtype, P): split runs with a workspace, the
    # unsplit kernel, fine lane cuts, fp32, and more sequences than the listed
    # split takes (partition items, with a separate token write)
    (40, (100, 3000), 4, 4, 128, 16, "bf16", 256),
    (40, (100, 3000), 4, 4, 128, 16, "bf16", 0),
    (300, (100, 2000), 4, 2, 128, 16, "bf16", 256),
    (30, (1, 700), 8, 2, 64, 32, "f32", 64),
    (25, (1, 400), 1, 4, 128, 32, "bf16", 32),
    (4200, (1, 90), 2, 2, 64, 16, "bf16", 32),
]


@pytest.mark.parametrize("case", range(len(DECODE_STEP_CASES)))
def test_decode_step_equals_separate_calls(case):
    # pkv_decode_step (token write inside the attention call) gives the bits of
    # pkv_reshape_and_cache followed by pkv_paged_attention_decode: the same
    # output and the same caches, starting from caches whose decode slots hold NaN
    GpuBatch = runner()
    nseq, lens, G, Hkv, d, B, dt, P = DECODE_STEP_CASES[case]
    say(f"case {case}: S={nseq} lens={lens} G={G} Hkv={Hkv} d={d} B={B} {dt} P={P}")
    w = wl.small_decode(nseq, lens, G * Hkv, Hkv, d, B, dt, seed=31 + case)
    gb = GpuBatch(w)
    assert gb.decode_rows_match
    ref = gb.step_separate(P).clone()
    k0, v0 = cache_bits(gb.k_cache).clone(), cache_bits(gb.v_cache).clone()
    for i in range(2):
        poison_decode_slots(gb)
        assert not torch.equal(cache_bits(gb.k_cache), k0)
        gb.out.fill_(float("nan"))
        gb.step(P)
        torch.cuda.synchronize()
        assert torch.equal(cache_bits(gb.k_cache), k0), i
        assert torch.equal(cache_bits(gb.v_cache), v0), i
        assert torch.equal(gb.out, ref), i


@pytest.mark.parametrize("name", ["llama7b_bf16", "gqa_bf16_b16", "gqa_bf16_b32", "beam_cow_bf16", "long_bf16"])
def test_decode_step_named_full_size(name):
    # the benchmarked step at full size, copy-on-write forks included: the
    # fused call writes every new token and matches the separate calls bitwise
    GpuBatch = runner()
    w = wl.named(name, seed=5)
    say(f"case {name}: S={w.num_seqs} max_n={w.max_context_len}")
    gb = GpuBatch(w)
    assert gb.decode_rows_match
    P = w.spec.partition_size
    ref = gb.step_separate(P).clone()
    k0, v0 = cache_bits(gb.k_cache).clone(), cache_bits(gb.v_cache).clone()
    poison_decode_slots(gb)
    gb.out.fill_(float("nan"))
    gb.step(P)
    torch.cuda.synchronize()
    assert torch.equal(cache_bits(gb.k_cache), k0)
    assert torch.equal(cache_bits(gb.v_cache), v0)
    assert torch.equal(gb.out, ref)


@pytest.mark.parametrize("nseq", [5, 4100])
def test_decode_step_skips_bad_sequences(nseq):
    # a sequence with a zero, negative or too-long length, or whose last block
    # id is out of range, gets no token write; the others are written as usual
    import paged_kv_cache_physical_amd as pk
    GpuBatch = runner()
    w = wl.small_decode(nseq, (40, 300), 8, 2, 128, 16, "bf16", seed=4)
    gb = GpuBatch(w)
    ref = gb.step_separate(64).cpu().numpy()
    good_k, good_v = cache_bits(gb.k_cache).clone(), cache_bits(gb.v_cache).clone()
    poison_decode_slots(gb)
    # the expected caches: the four bad sequences keep their poisoned slots
    d = gb.decode
    bad_rows = [0, 1, 2, 3]
    keep = torch.ones(nseq, dtype=torch.bool, device="cuda")
    keep[bad_rows] = False
    kc, vc = gb.k_cache.clone(), gb.v_cache.clone()
    pk.pkv_reshape_and_cache(d.k_new[keep].contiguous(), d.v_new[keep].contiguous(), kc, vc,
                             d.slots[keep].contiguous(), 16)
    exp_k, exp_v = cache_bits(kc), cache_bits(vc)
    lens = gb.context_lens.clone()
    bad_lens = lens.clone()
    bad_lens[0], bad_lens[1], bad_lens[2] = 0, -3, gb.max_context_len + 1
    gb.context_lens.copy_(bad_lens)
    tables = gb.block_tables.clone()
    bad_tables = tables.clone()
    bad_tables[3, (int(lens[3]) - 1) // 16] = w.num_blocks
    gb.block_tables.copy_(bad_tables)
    gb.out.fill_(float("nan"))
    gb.step(64)
    torch.cuda.synchronize()
    assert torch.equal(cache_bits(gb.k_cache), exp_k)
    assert torch.equal(cache_bits(gb.v_cache), exp_v)
    out = gb.out.cpu().numpy()
    assert np.all(out[0] == 0)
    assert np.all(np.isnan(out[1:4]))
    np.testing.assert_array_equal(out[4:], ref[4:])
    gb.context_lens.copy_(lens)
    gb.block_tables.copy_(tables)
    gb.step(64)
    torch.cuda.synchronize()
    assert torch.equal(cache_bits(gb.k_cache), good_k) and torch.equal(cache_bits(gb.v_cache), good_v)
    np.testing.assert_array_equal(gb.out.cpu().numpy(), ref)


def test_edge_lengths_and_bad_inputs():
    GpuBatch = runner()
    w = wl.small_decode(5, (40, 300), 8, 2, 128, 16, "bf16", seed=4)
    gb = GpuBatch(w)
    refs = {P: gb.attention(P).cpu().numpy().copy() for P in (0, 16, 64)}
    lens = gb.context_lens.clone()
    tables = gb.block_tables.clone()
    # a zero-length sequence gives zeros; lengths past max_context_len or negative give NaN
    gb.context_lens.copy_(torch.tensor([0, -3, gb.max_context_len + 1, int(lens[3]), int(lens[4])],
                                       dtype=torch.int32, device="cuda"))
    for P in (0, 64):
        out = gb.attention(P).cpu().numpy()
        assert np.all(out[0] == 0)
        assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
        np.testing.assert_array_equal(out[3:], refs[P][3:])
    gb.context_lens.copy_(lens)
    # an out-of-range block id poisons only its own sequence
    bad = tables.clone()
    bad[2, 1] = w.num_blocks
    gb.block_tables.copy_(bad)
    for P in (0, 16):
        out = gb.attention(P).cpu().numpy()
        assert np.all(np.isnan(out[2]))
        np.testing.assert_array_equal(np.delete(out, 2, axis=0), np.delete(refs[P], 2, axis=0))
    gb.block_tables.copy_(tables)
    np.testing.assert_array_equal(gb.attention(64).cpu().numpy(), refs[64])


def test_reshape_skips_negative_and_out_of_range_slots():
    import paged_kv_cache_physical_amd as pk
    nb, H, B, d = 4, 2, 16, 128
    kc, vc = pk.empty_caches(nb, H, B, d, "bf16")
    kcn, vcn = oc.empty_caches(nb, H, B, d, "bf16")
    rng = np.random.default_rng(0)
    k = wl.draw_values(rng, (4, H, d), "bf16")
    v = wl.draw_values(rng, (4, H, d), "bf16")
    slots = np.array([5, -1, nb * B, 63], np.int64)
    from paged_kv_cache_physical_amd.runner import _to_device
    pk.pkv_reshape_and_cache(_to_device(k, "bf16", "cuda"), _to_device(v, "bf16", "cuda"), kc, vc,
                             torch.from_numpy(slots).cuda(), B)
    keep = np.array([0, 3])
    oc.scatter(kcn, vcn, k[keep], v[keep], slots[keep])
    assert same_bits(host_bits(kc), kcn)
    assert same_bits(host_bits(vc), vcn)


def test_copy_blocks_f32_exact():
    import paged_kv_cache_physical_amd as pk
    nb, H, B, d = 6, 4, 32, 64
    kc, vc = pk.empty_caches(nb, H, B, d, "f32")
    kc.copy_(torch.randn_like(kc))
    vc.copy_(torch.randn_like(vc))
    k0, v0 = kc.cpu().numpy(), vc.cpu().numpy()
    pairs = np.array([[1, 4], [3, 0], [2, 9]], np.int32)  # the last pair is out of range: skipped
    pk.pkv_copy_blocks(kc, vc, torch.from_numpy(pairs).cuda())
    kn, vn = k0.copy(), v0.copy()
    oc.copy_blocks(kn, vn, pairs[:2])
    assert same_bits(kc.cpu().numpy(), kn) and same_bits(vc.cpu().numpy(), vn)


def test_empty_batch_is_noop():
    import paged_kv_cache_physical_amd as pk
    kc, vc = pk.empty_caches(2, 1, 16, 64, "f32")
    q = torch.empty((0, 1, 64), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    pk.pkv_paged_attention_decode(out, q, kc, vc, torch.empty((0, 1), dtype=torch.int32, device="cuda"),
                                  torch.empty(0, dtype=torch.int32, device="cuda"), 0, 0.125, 0)
    torch.cuda.synchronize()
