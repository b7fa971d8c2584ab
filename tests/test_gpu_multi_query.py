"""GPU parity of runs of causal queries (pkv_paged_attention_multi) against the
float64 oracle, through the C-ABI: whole prompts, short runs over long
contexts, the uncached rest of prefix-cached prompts, and speculative
verification followed by a rollback (pkv_seq_truncate) and a decode step.

Bars as for decode: fp32 max abs <= 1e-5; bf16 max abs <= 1e-2 and relative
L2 <= 2e-3; every case also relative L2 <= 1e-4."""

import numpy as np
import pytest

import workloads as wl
from oracle import allocator as al
from oracle import attention as oa
from oracle import cache as oc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu(libpkv):
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def to_dev(a, dt):
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def check_close(out, ref, dt, what):
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = float(np.max(np.abs(out - ref)))
    rl2 = float(np.linalg.norm(out - ref) / np.linalg.norm(ref))
    say(f"  {what}: max_abs={err:.3e} rel_l2={rl2:.3e}")
    if dt == "f32":
        assert err <= 1e-5, (what, err)
    else:
        assert err <= 1e-2 and rl2 <= 2e-3, (what, err, rl2)
    assert rl2 <= 1e-4, (what, rl2)


class Batch:
    """Sequences of given lengths written through the C pool (GPU caches) and the oracle pool (host caches)."""

    def __init__(self, lens, Hq, Hkv, d, B, dt, seed, spare=8):
        import paged_kv_cache_physical_amd as pk
        self.pk, self.lens, self.Hq, self.Hkv, self.d, self.B, self.dt = pk, list(lens), Hq, Hkv, d, B, dt
        self.seed = seed
        nb = sum(-(-n // B) for n in lens) + spare
        order = wl.rng_for(seed, wl.STREAM_PERM).permutation(nb).astype(np.int32)
        self.nb = nb
        self.pool, self.opool = pk.Pool(nb, B, order), al.BlockPool(nb, B, order)
        self.caches = pk.empty_caches(nb, Hkv, B, d, dt)
        self.ocaches = oc.empty_caches(nb, Hkv, B, d, dt)
        self.ids = [self.pool.create() for _ in lens]
        assert self.ids == [self.opool.create() for _ in lens]
        self.k = [wl.draw_values(wl.rng_for(seed, wl.STREAM_KV, i, 0), (n, Hkv, d), dt) for i, n in enumerate(lens)]
        self.v = [wl.draw_values(wl.rng_for(seed, wl.STREAM_KV, i, 1), (n, Hkv, d), dt) for i, n in enumerate(lens)]
        self.write(list(range(len(lens))), [0] * len(lens), list(lens))

    def write(self, which, starts, counts):
        """Append counts[j] tokens to sequence which[j] (positions starts[j]...) and write their K/V on both sides."""
        seqs = [self.ids[i] for i in which]
        slots, pairs = self.pool.append(seqs, counts)
        oslots, opairs = self.opool.append(seqs, counts)
        assert np.array_equal(slots, oslots) and np.array_equal(pairs, opairs)
        if len(pairs):
            self.pk.pkv_copy_blocks(*self.caches, torch.from_numpy(pairs).cuda())
            oc.copy_blocks(*self.ocaches, opairs)
        k = np.concatenate([self.k[i][s:s + c] for i, s, c in zip(which, starts, counts)])
        v = np.concatenate([self.v[i][s:s + c] for i, s, c in zip(which, starts, counts)])
        self.pk.pkv_reshape_and_cache(to_dev(k, self.dt), to_dev(v, self.dt), *self.caches,
                                      torch.from_numpy(slots).cuda(), self.B)
        oc.scatter(*self.ocaches, k, v, oslots)

    def tables(self):
        mb = max(1, max(-(-self.pool.length(i) // self.B) for i in self.ids))
        t, l = self.pool.block_tables(self.ids, mb)
        ot, ol = self.opool.block_tables(self.ids, mb)
        assert np.array_equal(t, ot) and np.array_equal(l, ol)
        return t, l

    def multi(self, runs, q, tables=None, lens=None, query_start=None, max_query_len=None, out=None, split=False,
              order=None, scale=None):
        t, l = self.tables() if tables is None else (tables, lens)
        starts = np.concatenate([[0], np.cumsum(runs)]).astype(np.int32) if query_start is None else query_start
        T = q.shape[0]
        out = torch.full((T, self.Hq, self.d), float("nan"), dtype=torch.float32, device="cuda") if out is None else out
        mql = int(max(runs) if max_query_len is None else max_query_len)
        ws = None
        if split:
            nbytes = self.pk.pkv_attention_multi_workspace_bytes(len(l), self.Hq, self.Hkv, self.d, int(max(l.max(), 1)),
                                                                 mql)
            assert nbytes > 0, "the plan does not split this batch"
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.pk.pkv_paged_attention_multi(out, to_dev(q, self.dt), *self.caches, torch.from_numpy(t).cuda(),
                                          torch.from_numpy(l).cuda(), torch.from_numpy(starts).cuda(),
                                          int(max(l.max(), 1)), mql,
                                          1.0 / np.sqrt(self.d) if scale is None else scale, workspace=ws,
                                          seq_order=None if order is None else torch.tensor(order, dtype=torch.int32,
                                                                                            device="cuda"))
        torch.cuda.synchronize()
        return out.cpu().numpy(), t, l, starts

    def oracle(self, q, t, l, starts, scale=None):
        sc = np.float32(1.0 / np.sqrt(self.d) if scale is None else scale)
        return oa.paged_attention_multi(q, *self.ocaches, t, l, starts, sc, self.dt)


GRID = [(dt, d, G, B) for dt in ("f32", "bf16") for d in (64, 128) for G in (1, 2, 4, 8) for B in (16, 32)]


@pytest.mark.parametrize("tiles", ["auto", "2"])
@pytest.mark.parametrize("dt,d,G,B", GRID)
def test_runs_grid(dt, d, G, B, tiles, monkeypatch):
    """Every supported shape; "2" forces two row tiles per wave (PKV_MULTI_TILES), which these small batches would
    not choose, so both kernels of each shape are checked."""
    if tiles != "auto":
        monkeypatch.setenv("PKV_MULTI_TILES", tiles)
    rng = wl.rng_for(G * 100 + d + B, 99)
    lens = [int(x) for x in rng.integers(1, 300, size=6)] + [1, 17]
    runs = [n if i % 3 == 0 else int(rng.integers(1, min(n, 40) + 1)) for i, n in enumerate(lens)]
    runs[-1] = 17  # a whole 17-token prompt
    Hkv = 2
    say(f"case {dt} d={d} G={G} B={B} tiles={tiles}: lens={lens} runs={runs}")
    b = Batch(lens, G * Hkv, Hkv, d, B, dt, seed=G + d + B)
    q = wl.draw_values(wl.rng_for(5, wl.STREAM_Q, G, d), (sum(runs), G * Hkv, d), dt)
    out, t, l, starts = b.multi(runs, q)
    check_close(out, b.oracle(q, t, l, starts), dt, "runs")


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("dt,scale", [(dt, x) for dt in ("bf16", "f32") for x in (-0.125, 0.0, 0.3)] +
                         [("bf16", 0.6), ("bf16", -1.5)])
def test_scale_sign_and_size(dt, scale, split):
    """Any finite scale: a negative one (the queries enter with flipped signs), zero (equal weights over the visible
    tokens) and larger ones, whose logits spread over tens of exp2 units, so that the row references move many
    times and the weights of a chunk reach up to 2^8 between moves; with and without context splits.  (fp32 keeps
    to scales whose logits' float32 rounding stays inside its 1e-5 bound.)"""
    if split:
        lens, runs = [1200, 700, 64], [3, 2, 1]  # few rows per pair over long contexts: the plan splits them
    else:
        lens, runs = [300, 47, 513, 96], [300, 5, 200, 1]
    b = Batch(lens, 8, 2, 128, 16, dt, seed=77)
    q = wl.draw_values(wl.rng_for(11, wl.STREAM_Q), (sum(runs), 8, 128), dt)
    say(f"case {dt} scale={scale} split={split}")
    out, t, l, starts = b.multi(runs, q, split=split, scale=scale)
    check_close(out, b.oracle(q, t, l, starts, scale=scale), dt, f"scale {scale}")


@pytest.mark.parametrize("dt,B", [("bf16", 16), ("f32", 32)])
def test_whole_prompts_long(dt, B):
    """Prompt attention over 1000-2000 tokens: many chunks and many row tiles per (sequence, KV head)."""
    lens = [1500, 2048, 1001]
    b = Batch(lens, 32, 8, 128, B, dt, seed=21)
    q = wl.draw_values(wl.rng_for(6, wl.STREAM_Q), (sum(lens), 32, 128), dt)
    out, t, l, starts = b.multi(lens, q)
    check_close(out, b.oracle(q, t, l, starts), dt, "whole prompts")


@pytest.mark.parametrize("dt,B", [("bf16", 16), ("bf16", 32), ("f32", 16)])
def test_prefix_cached_prompts_compute_only_their_tails(dt, B):
    """Requests that share stems take their leading blocks from the prefix cache; the multi-query call over just
    the uncached tokens gives the rows of each whole prompt's causal attention."""
    import paged_kv_cache_physical_amd as pk
    R, Hq, Hkv, d = 16, 32, 8, 128
    pr = wl.PrefixRequests(seed=40 + B, num_requests=R, num_stems=3, stem_range=(100, 700), tail_range=(1, 120),
                           num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, kv_dtype=dt)
    lens = [len(pr.prompt(r)) for r in range(R)]
    nb = sum(-(-n // B) for n in lens) + 16
    order = wl.rng_for(8, wl.STREAM_PERM).permutation(nb).astype(np.int32)
    pool = pk.Pool(nb, B, order)
    caches = pk.empty_caches(nb, Hkv, B, d, dt)
    ids, runs = [], []
    for r in range(R):
        ids_r = pr.prompt(r)
        sid, hit = pool.create_prefixed(ids_r)
        slots, pairs = pool.append([sid], [len(ids_r) - hit], token_ids=ids_r[hit:])
        assert pairs.shape == (0, 2)
        k, v = pr.kv(r)
        pk.pkv_reshape_and_cache(to_dev(k[hit:], dt), to_dev(v[hit:], dt), *caches, torch.from_numpy(slots).cuda(), B)
        ids.append(sid)
        runs.append(len(ids_r) - hit)
    assert sum(runs) < sum(lens) // 2, (sum(runs), sum(lens))
    mb = max(-(-n // B) for n in lens)
    t, l = pool.block_tables(ids, mb)
    # one query per prompt position; the call gets only the uncached positions' rows
    qfull = [wl.draw_values(wl.rng_for(9, wl.STREAM_Q, r), (lens[r], Hq, d), dt) for r in range(R)]
    q = np.concatenate([qf[n - k:] for qf, n, k in zip(qfull, lens, runs)])
    starts = np.concatenate([[0], np.cumsum(runs)]).astype(np.int32)
    out = torch.full((q.shape[0], Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    pk.pkv_paged_attention_multi(out, to_dev(q, dt), *caches, torch.from_numpy(t).cuda(), torch.from_numpy(l).cuda(),
                                 torch.from_numpy(starts).cuda(), int(l.max()), max(runs), 1.0 / np.sqrt(d))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    scale = np.float32(1.0 / np.sqrt(d))
    ref = []
    for r in range(R):  # each prompt's own contiguous K/V, never read through a cache
        k, v = (oc.to_f64(x, dt) for x in pr.kv(r))
        qq = oc.to_f64(qfull[r], dt)
        for p in range(lens[r] - runs[r], lens[r]):
            ref.append(oa.attention_contiguous(qq[p], k[:p + 1], v[:p + 1], scale))
    check_close(out, np.stack(ref), dt, "prefix-cached tails")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_speculative_verify_rollback_decode(dt):
    """Stage k drafted tokens, verify them with one multi-query call, keep a prefix, roll back the rest, write the
    corrected token and decode: every step against the oracle, and the pool against the oracle pool."""
    import paged_kv_cache_physical_amd as pk
    B, Hq, Hkv, d, kdraft = 16, 32, 8, 128, 5
    rng = wl.rng_for(77, 1)
    base = [int(x) for x in rng.integers(20, 600, size=12)]
    total = [n + kdraft for n in base]
    b = Batch(total, Hq, Hkv, d, B, dt, seed=13, spare=32)
    # the batch holds base + drafted tokens already; the drafts are the last kdraft positions
    runs = [kdraft] * len(base)
    q = wl.draw_values(wl.rng_for(14, wl.STREAM_Q), (sum(runs), Hq, d), dt)
    out, t, l, starts = b.multi(runs, q)
    check_close(out, b.oracle(q, t, l, starts), dt, "verify")
    # keep a different number of drafts per sequence, drop the rest
    keep = [int(x) for x in rng.integers(0, kdraft + 1, size=len(base))]
    for i, (n, kk) in enumerate(zip(base, keep)):
        b.pool.truncate(b.ids[i], n + kk)
        b.opool.truncate(b.ids[i], n + kk)
    b.pool.validate()
    assert b.pool.free_list().tolist() == b.opool.free_list()
    # the corrected token: new K/V at position n + keep
    for i, (n, kk) in enumerate(zip(base, keep)):
        b.k[i] = np.concatenate([b.k[i][:n + kk], wl.draw_values(wl.rng_for(15, i, 0), (1, Hkv, d), dt)])
        b.v[i] = np.concatenate([b.v[i][:n + kk], wl.draw_values(wl.rng_for(15, i, 1), (1, Hkv, d), dt)])
    b.write(list(range(len(base))), [n + kk for n, kk in zip(base, keep)], [1] * len(base))
    t, l = b.tables()
    assert l.tolist() == [n + kk + 1 for n, kk in zip(base, keep)]
    qd = wl.draw_values(wl.rng_for(16, wl.STREAM_Q), (len(base), Hq, d), dt)
    out, *_ = b.multi([1] * len(base), qd, tables=t, lens=l)
    ref = oa.paged_attention(qd, *b.ocaches, t, l, np.float32(1.0 / np.sqrt(d)), dt)
    check_close(out, ref, dt, "decode after rollback")
    # the decode kernel agrees with the one-query runs
    od = torch.empty((len(base), Hq, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(pk.pkv_attention_workspace_bytes(len(base), Hq, Hkv, d, B, int(l.max()), 0), 1),
                     dtype=torch.uint8, device="cuda")
    pk.pkv_paged_attention_decode(od, to_dev(qd, dt), *b.caches, torch.from_numpy(t).cuda(), torch.from_numpy(l).cuda(),
                                  int(l.max()), 1.0 / np.sqrt(d), 0, ws)
    torch.cuda.synchronize()
    check_close(od.cpu().numpy(), ref, dt, "decode kernel")


def test_edge_cases():
    """Empty runs, runs that cannot be computed (NaN rows), runs outside the rows (untouched), bad block ids."""
    b = Batch([40, 33, 20, 64, 9], 8, 2, 64, 16, "f32", seed=3)
    t, l = b.tables()
    # sequence 1: empty run; sequence 2: a run longer than its context (NaN); sequence 4: longer than max_query_len
    runs = [3, 0, 21, 2, 9]
    T = sum(runs)
    q = wl.draw_values(wl.rng_for(4, wl.STREAM_Q), (T, 8, 64), "f32")
    starts = np.concatenate([[0], np.cumsum(runs)]).astype(np.int32)
    sentinel = torch.full((T, 8, 64), 7.0, dtype=torch.float32, device="cuda")
    out, *_ = b.multi(runs, q, tables=t, lens=l, query_start=starts, max_query_len=8, out=sentinel)
    ref = b.oracle(q[:3], t[:1], l[:1], starts[:2])
    check_close(out[:3], ref, "f32", "sequence 0")
    assert np.all(np.isnan(out[3:3 + 8]))  # q_s > max_query_len and > n_s: the covered rows say so
    assert np.all(out[3 + 8:24] == 7.0)  # rows past max_query_len are not written
    ref3 = b.oracle(q[24:26], t[3:4], l[3:4], np.array([0, 2], np.int32))
    check_close(out[24:26], ref3, "f32", "sequence 3")
    assert np.all(np.isnan(out[26:26 + 8])) and np.all(out[26 + 8:] == 7.0)
    # a bad block id poisons only its sequence; a run outside [0, T) is left alone
    t2 = t.copy()
    t2[3, 1] = b.nb + 5
    starts2 = np.array([0, 3, 3, 3, 5, T + 4], np.int32)
    runs2 = [3, 0, 0, 2, 1]
    sentinel.fill_(7.0)
    out, *_ = b.multi(runs2, q, tables=t2, lens=l, query_start=starts2, out=sentinel)
    check_close(out[:3], ref, "f32", "sequence 0 again")
    assert np.all(np.isnan(out[3:5])) and np.all(out[5:] == 7.0)
    # an empty call does nothing
    b.pk.pkv_paged_attention_multi(sentinel[:0], to_dev(q[:0], "f32"), *b.caches, torch.from_numpy(t).cuda(),
                                   torch.from_numpy(l).cuda(), torch.zeros(6, dtype=torch.int32, device="cuda"),
                                   64, 0, 0.125)
    torch.cuda.synchronize()


@pytest.mark.parametrize("tiles", ["1", "2"])
def test_edge_cases_wide_runs(tiles, monkeypatch):
    """The edge cases with more than 64 rows per (sequence, KV head), in both kernels: runs longer than
    max_query_len or than their context give NaN on the rows the launch covers and leave the rest alone, an empty
    run writes nothing, and a bad block id poisons only the rows of its own sequence."""
    monkeypatch.setenv("PKV_MULTI_TILES", tiles)
    b = Batch([40, 33, 20, 64, 90], 8, 2, 64, 16, "f32", seed=3)  # G = 4: max_query_len 20 makes 80 rows
    t, l = b.tables()
    runs = [30, 0, 21, 2, 20]
    T = sum(runs)
    q = wl.draw_values(wl.rng_for(41, wl.STREAM_Q), (T, 8, 64), "f32")
    starts = np.concatenate([[0], np.cumsum(runs)]).astype(np.int32)
    sentinel = torch.full((T, 8, 64), 7.0, dtype=torch.float32, device="cuda")
    out, *_ = b.multi(runs, q, tables=t, lens=l, query_start=starts, max_query_len=20, out=sentinel)
    assert np.all(np.isnan(out[0:20])) and np.all(out[20:30] == 7.0)  # 30 > max_query_len
    assert np.all(np.isnan(out[30:50])) and np.all(out[50] == 7.0)  # 21 > its 20-token context
    ref3 = b.oracle(q[51:53], t[3:4], l[3:4], np.array([0, 2], np.int32))
    ref4 = b.oracle(q[53:73], t[4:5], l[4:5], np.array([0, 20], np.int32))
    check_close(out[51:53], ref3, "f32", f"sequence 3, tiles {tiles}")
    check_close(out[53:73], ref4, "f32", f"sequence 4, tiles {tiles}")
    t2 = t.copy()
    t2[4, 2] = b.nb + 5  # tokens 32-47 of sequence 4: every one of its rows sees them
    sentinel.fill_(7.0)
    out, *_ = b.multi(runs, q, tables=t2, lens=l, query_start=starts, max_query_len=20, out=sentinel)
    check_close(out[51:53], ref3, "f32", f"sequence 3 beside a bad id, tiles {tiles}")
    assert np.all(np.isnan(out[53:73]))


@pytest.mark.parametrize("split", [False, True])
def test_bad_block_id_in_the_second_half_of_a_chunk(split):
    """bf16, d = 64, B = 16: a 32-token chunk is staged by two halves of the workgroup, waves 0-1 loading tokens
    0-15 and waves 2-3 tokens 16-31, while every wave reads the whole chunk from LDS.  A bad block id in tokens
    16-31 must make the rows that saw it NaN even when all of them sit in wave 0 (3 queries x G = 4 rows), with
    and without context splits; the other sequence stays exact."""
    lens = [1200, 700]
    runs = [3, 3]
    b = Batch(lens, 8, 2, 64, 16, "bf16", seed=51)
    t, l = b.tables()
    q = wl.draw_values(wl.rng_for(52, wl.STREAM_Q), (sum(runs), 8, 64), "bf16")
    out, _, _, starts = b.multi(runs, q, tables=t, lens=l, split=split)
    ref = b.oracle(q, t, l, starts)
    check_close(out, ref, "bf16", f"both sequences, split={split}")
    t2 = t.copy()
    t2[0, 1] = b.nb + 5  # block 1 of sequence 0: tokens 16-31, the second half of its first chunk
    out, *_ = b.multi(runs, q, tables=t2, lens=l, split=split)
    assert np.all(np.isnan(out[:3])), "rows that read a bad block id"
    check_close(out[3:], ref[3:], "bf16", f"the sequence beside it, split={split}")


def test_full_size_prefill(monkeypatch):
    """Whole prompts at the prefill shape (16 prompts x 2048 tokens, 32/8 heads, d 128, bf16, B 16): the batch's
    rows fill the GPU, so the call takes two row tiles per wave.  Every row of four whole prompts (first, last and
    two between) against the float64 oracle over the oracle pool's own caches; forcing one tile per wave gives the
    same bits for the whole batch."""
    S, L, Hq, Hkv, d = 16, 2048, 32, 8, 128
    monkeypatch.delenv("PKV_MULTI_TILES", raising=False)
    b = Batch([L] * S, Hq, Hkv, d, 16, "bf16", seed=23)
    q = wl.draw_values(wl.rng_for(24, wl.STREAM_Q), (S * L, Hq, d), "bf16")
    out2, t, l, starts = b.multi([L] * S, q)
    for i in (0, 5, 10, 15):
        rows = slice(starts[i], starts[i + 1])
        ref = b.oracle(q[rows], t[i:i + 1], l[i:i + 1], np.array([0, L], np.int32))
        check_close(out2[rows], ref, "bf16", f"prompt {i}, all {L} rows")
    monkeypatch.setenv("PKV_MULTI_TILES", "1")
    out1, _, _, _ = b.multi([L] * S, q)
    assert np.array_equal(out1, out2), float(np.max(np.abs(out1 - out2)))


def test_full_size_verification():
    """Speculative verification at the Llama-7B decode shape (64 sequences, 32 heads, d 128, bf16, lengths
    uniform in [128, 2048]) with 4 drafted tokens per sequence: every row of the batch against the oracle."""
    w = wl.named("llama7b_bf16", seed=0)
    s = w.spec
    runs = [4] * w.num_seqs
    lens = [int(n) for n in w.context_lens]
    b = Batch(lens, s.num_q_heads, s.num_kv_heads, s.head_dim, s.block_size, s.kv_dtype, seed=0, spare=64)
    q = wl.draw_values(wl.rng_for(17, wl.STREAM_Q), (sum(runs), s.num_q_heads, s.head_dim), s.kv_dtype)
    out, t, l, starts = b.multi(runs, q)
    check_close(out, b.oracle(q, t, l, starts), s.kv_dtype, f"all {len(runs)} runs")


def test_full_size_mixed_step(monkeypatch):
    """One continuous-batching step at full size, launched as timed (with a workspace, longest-first order): 64
    sequences with contexts uniform in [640, 2048], 32/8 heads, d 128, bf16, B 16; 4 of them take a 512-query
    prompt chunk and 60 decode one token.  The decodes go to the decode kernel's pass, the chunks to the runs
    kernel; every row (the four chunks and the 60 decodes) against the oracle, and again with every run on the
    runs kernel (PKV_MULTI_PATH=runs)."""
    rng = wl.rng_for(31, 0)
    S, Hq, Hkv, d = 64, 32, 8, 128
    lens = [int(x) for x in rng.integers(640, 2048, size=S, endpoint=True)]
    runs = [512] * 4 + [1] * (S - 4)
    b = Batch(lens, Hq, Hkv, d, 16, "bf16", seed=31)
    q = wl.draw_values(wl.rng_for(32, wl.STREAM_Q), (sum(runs), Hq, d), "bf16")
    order = np.argsort(-np.array(lens), kind="stable").astype(np.int32)
    out, t, l, starts = b.multi(runs, q, order=order, split=True)
    ref = b.oracle(q, t, l, starts)
    check_close(out[:4 * 512], ref[:4 * 512], "bf16", "the four prompt chunks, all rows")
    check_close(out[4 * 512:], ref[4 * 512:], "bf16", "the 60 decodes")
    monkeypatch.setenv("PKV_MULTI_PATH", "runs")
    other, *_ = b.multi(runs, q, order=order, split=True)
    check_close(other[:4 * 512], ref[:4 * 512], "bf16", "the four prompt chunks, runs kernel only")
    check_close(other[4 * 512:], ref[4 * 512:], "bf16", "the 60 decodes, runs kernel only")
    assert np.array_equal(other[:4 * 512], out[:4 * 512])  # the chunks come from the runs kernel either way


MIXED_GRID = [("bf16", 128, 4, 16), ("f32", 64, 8, 32), ("bf16", 64, 1, 32), ("f32", 128, 2, 16),
              ("bf16", 128, 8, 32)]


@pytest.mark.parametrize("dt,d,G,B", MIXED_GRID)
def test_mixed_step_two_launches(dt, d, G, B, monkeypatch):
    """A batch whose longest run is longer than 16 / G queries while other runs are shorter (prompt chunks and a
    whole prompt beside decodes and short verifications) takes two launches when given a workspace: the runs of
    at most 16 / G queries on the decode kernel's pass, over contexts cut into 512-token partitions, the longer
    ones on the runs kernel.  Every row against the oracle; the runs kernel alone (PKV_MULTI_PATH=runs) gives the
    long runs' rows bit for bit and the short ones within the same bars."""
    k = 16 // G
    lens = [1800, 700, 2500, 64, 1200, 1, 900, 3000, 40, 513]
    runs = [1, k, 200, 1, k + 1, 1, min(2, k), 1, 40, 1]
    Hkv = 2
    say(f"case {dt} d={d} G={G} B={B}: k={k} runs={runs}")
    b = Batch(lens, G * Hkv, Hkv, d, B, dt, seed=G + d + B + 91)
    q = wl.draw_values(wl.rng_for(92, wl.STREAM_Q, G, d), (sum(runs), G * Hkv, d), dt)
    out, t, l, starts = b.multi(runs, q, split=True)
    ref = b.oracle(q, t, l, starts)
    check_close(out, ref, dt, "two launches")
    monkeypatch.setenv("PKV_MULTI_PATH", "runs")
    other, *_ = b.multi(runs, q, split=True)
    check_close(other, ref, dt, "runs kernel only")
    long_rows = np.concatenate([np.arange(starts[i], starts[i + 1]) for i, r in enumerate(runs) if r > k])
    assert np.array_equal(other[long_rows], out[long_rows])


def test_mixed_step_two_launches_edges():
    """The runs kernel's contract holds across the two launches (G = 4, max_query_len 12: runs of up to 4 queries
    on the decode kernel's pass, longer ones on the runs kernel): an empty run writes nothing; a run longer than
    its context gives NaN rows, on either launch; a run longer than max_query_len gives NaN on its first
    max_query_len rows and leaves the rest alone; a bad block id poisons only its own sequence, a short run over
    a cut context or a prompt."""
    lens = [1400, 33, 20, 640, 9, 2100, 700, 2, 0, 3]
    runs = [3, 0, 21, 2, 9, 4, 1, 3, 1, 5]
    b = Batch(lens, 8, 2, 64, 16, "f32", seed=93)
    t, l = b.tables()
    T = sum(runs)
    q = wl.draw_values(wl.rng_for(94, wl.STREAM_Q), (T, 8, 64), "f32")
    starts = np.concatenate([[0], np.cumsum(runs)]).astype(np.int32)
    rows = lambda i: slice(int(starts[i]), int(starts[i + 1]))
    sentinel = torch.full((T, 8, 64), 7.0, dtype=torch.float32, device="cuda")
    out, *_ = b.multi(runs, q, tables=t, lens=l, query_start=starts, max_query_len=12, out=sentinel, split=True)
    refs = {}
    for i in (0, 3, 4, 5, 6):
        refs[i] = b.oracle(q[rows(i)], t[i:i + 1], l[i:i + 1], np.array([0, runs[i]], np.int32))
        check_close(out[rows(i)], refs[i], "f32", f"sequence {i}")
    s2 = int(starts[2])
    assert np.all(np.isnan(out[s2:s2 + 12])) and np.all(out[s2 + 12:s2 + 21] == 7.0)  # 21 > 12 and > n: runs kernel
    assert np.all(np.isnan(out[rows(7)]))  # 3 > its 2-token context: decode kernel's pass
    assert np.all(np.isnan(out[rows(8)]))  # a decode with no context: decode kernel's pass
    assert np.all(np.isnan(out[rows(9)]))  # 5 > its 3-token context: runs kernel
    t2 = t.copy()
    t2[0, 40] = b.nb + 5  # a short run over a cut context
    t2[4, 0] = b.nb + 6   # the whole 9-token prompt
    sentinel.fill_(7.0)
    out, *_ = b.multi(runs, q, tables=t2, lens=l, query_start=starts, max_query_len=12, out=sentinel, split=True)
    assert np.all(np.isnan(out[rows(0)])) and np.all(np.isnan(out[rows(4)]))
    for i in (3, 5, 6):
        check_close(out[rows(i)], refs[i], "f32", f"sequence {i} beside bad ids")


@pytest.mark.parametrize("with_ws", [False, True])
def test_repeated_calls_and_graph_replays_are_bitwise_stable(with_ws):
    """Runs of queries give the same bits on every call, and as a captured HIP graph on every replay, with eager
    work and synchronisations between the replays; with a workspace the call takes two launches (the decode and
    the 3-query verification on the decode kernel's pass, the rest on the runs kernel)."""
    import paged_kv_cache_physical_amd as pk
    lens = [900, 1500, 37, 2048, 640, 1300]
    runs = [300, 7, 37, 512, 1, 3]
    b = Batch(lens, 32, 8, 128, 16, "bf16", seed=29)
    t, l = b.tables()
    q = to_dev(wl.draw_values(wl.rng_for(30, wl.STREAM_Q), (sum(runs), 32, 128), "bf16"), "bf16")
    starts = torch.from_numpy(np.concatenate([[0], np.cumsum(runs)]).astype(np.int32)).cuda()
    bt, cl = torch.from_numpy(t).cuda(), torch.from_numpy(l).cuda()
    out = torch.empty((sum(runs), 32, 128), dtype=torch.float32, device="cuda")
    ws = None
    if with_ws:
        nbytes = pk.pkv_attention_multi_workspace_bytes(len(lens), 32, 8, 128, int(l.max()), max(runs))
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    call = lambda: pk.pkv_paged_attention_multi(out, q, *b.caches, bt, cl, starts, int(l.max()), max(runs),
                                                1.0 / np.sqrt(128), stream=s, workspace=ws)
    with torch.cuda.stream(s):
        call()
        torch.cuda.synchronize()
        first = out.clone()
        assert bool(torch.isfinite(first).all())
        for i in range(6):
            out.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
            assert torch.equal(out, first), i
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call()
        for i in range(4):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, first), i
            out.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
            assert torch.equal(out, first), i



LISTED_GRID = [(dt, d, G, B) for dt in ("f32", "bf16") for d in (64, 128) for G in (1, 2, 4, 8) for B in (16, 32)]


@pytest.mark.parametrize("dt,d,G,B", LISTED_GRID)
def test_short_runs_on_the_decode_kernel(dt, d, G, B, monkeypatch):
    """Runs of at most 16 / G queries with a workspace take the decode kernel's listed path, the queries of a run
    as further matrix-core columns: every shape against the oracle, over contexts that are cut into 512-token
    partitions and between workgroups (runs of one query up to 16 / G, contexts from 1 to 3000 tokens), and the
    same rows from the runs kernel (PKV_MULTI_PATH=runs)."""
    import paged_kv_cache_physical_amd as pk
    k = 16 // G
    rng = wl.rng_for(500 + G * 10 + d + B, 2)
    lens = [int(x) for x in rng.integers(1, 3000, size=20)] + [1, 2, 513, 3000]
    runs = [min(n, int(x)) for n, x in zip(lens, rng.integers(1, k + 1, size=len(lens)))]
    runs[-1] = min(k, lens[-1])
    Hkv = 2
    say(f"case {dt} d={d} G={G} B={B}: k={k} runs={runs}")
    b = Batch(lens, G * Hkv, Hkv, d, B, dt, seed=G + d + B + 7)
    q = wl.draw_values(wl.rng_for(61, wl.STREAM_Q, G, d), (sum(runs), G * Hkv, d), dt)
    assert pk.pkv_attention_multi_workspace_bytes(len(lens), G * Hkv, Hkv, d, max(lens), max(runs)) > 0
    out, t, l, starts = b.multi(runs, q, split=True)
    ref = b.oracle(q, t, l, starts)
    check_close(out, ref, dt, "decode kernel")
    monkeypatch.setenv("PKV_MULTI_PATH", "runs")
    other, *_ = b.multi(runs, q, split=True)
    check_close(other, ref, dt, "runs kernel")


FOUR_GRID = [(dt, d, G, B) for dt in ("f32", "bf16") for d in (64, 128) for G in (1, 2) for B in (16, 32)]


@pytest.mark.parametrize("dt,d,G,B", FOUR_GRID)
def test_runs_of_up_to_four_queries_at_one_or_two_heads_per_kv_head(dt, d, G, B, monkeypatch):
    """With G <= 2 and runs of at most 4 queries the decode kernel's pass takes 4 queries per item (4 or 8
    matrix-core columns instead of the whole 16-column tile): every shape against the oracle over contexts cut
    into 512-token partitions and between workgroups, and against the runs kernel (PKV_MULTI_PATH=runs)."""
    rng = wl.rng_for(700 + G * 10 + d + B, 3)
    lens = [int(x) for x in rng.integers(1, 3000, size=20)] + [1, 3, 513, 3000]
    runs = [min(n, int(x)) for n, x in zip(lens, rng.integers(1, 5, size=len(lens)))]
    runs[-1] = 4
    Hkv = 2
    say(f"case {dt} d={d} G={G} B={B}: runs={runs}")
    b = Batch(lens, G * Hkv, Hkv, d, B, dt, seed=G + d + B + 17)
    q = wl.draw_values(wl.rng_for(71, wl.STREAM_Q, G, d), (sum(runs), G * Hkv, d), dt)
    out, t, l, starts = b.multi(runs, q, split=True)
    ref = b.oracle(q, t, l, starts)
    check_close(out, ref, dt, "decode kernel, 4 queries per item")
    monkeypatch.setenv("PKV_MULTI_PATH", "runs")
    other, *_ = b.multi(runs, q, split=True)
    check_close(other, ref, dt, "runs kernel")


ONE_QUERY_GRID = [("bf16", 128, 4, 16), ("f32", 64, 1, 32), ("bf16", 64, 8, 32), ("f32", 128, 2, 16)]


@pytest.mark.parametrize("dt,d,G,B", ONE_QUERY_GRID)
def test_one_query_runs_on_the_decode_kernel(dt, d, G, B):
    """Runs of one query each (max_query_len 1: decodes given as runs) on the decode kernel's listed pass, with
    the rows placed by query_start: every row against the oracle over contexts cut into 512-token partitions, with
    empty runs between them; a run over an empty context is NaN; a bad block id poisons only its sequence; a run
    outside the rows is left alone."""
    lens = [1800, 700, 2500, 64, 1200, 1, 900, 3000, 40, 513, 0]
    runs = [1, 1, 0, 1, 1, 1, 0, 1, 1, 1, 1]
    Hkv = 2
    b = Batch(lens, G * Hkv, Hkv, d, B, dt, seed=G + d + B + 95)
    t, l = b.tables()
    T = sum(runs)
    q = wl.draw_values(wl.rng_for(96, wl.STREAM_Q, G, d), (T, G * Hkv, d), dt)
    starts = np.concatenate([[0], np.cumsum(runs)]).astype(np.int32)
    sentinel = torch.full((T, G * Hkv, d), 7.0, dtype=torch.float32, device="cuda")
    out, *_ = b.multi(runs, q, tables=t, lens=l, query_start=starts, out=sentinel, split=True)
    live = [i for i in range(len(lens)) if runs[i] == 1 and lens[i] > 0]
    rows = np.array([starts[i] for i in live])
    ref = b.oracle(q[rows], t[live], l[live], np.arange(len(live) + 1, dtype=np.int32))
    check_close(out[rows], ref, dt, "one-query runs")
    assert np.all(np.isnan(out[starts[10]]))  # a query over no context
    t2 = t.copy()
    t2[7, 50] = b.nb + 5
    starts2 = starts.copy()
    starts2[10] = T + 3  # the run of sequence 9 now reaches past the rows: left alone
    sentinel.fill_(7.0)
    out, *_ = b.multi(runs, q, tables=t2, lens=l, query_start=starts2, max_query_len=1, out=sentinel, split=True)
    assert np.all(np.isnan(out[starts[7]]))
    assert np.all(out[starts[9]] == 7.0)
    keep = [j for j, i in enumerate(live) if i not in (7, 9)]
    check_close(out[rows[keep]], ref[keep], dt, "one-query runs beside a bad id")


def test_short_runs_on_the_decode_kernel_edges():
    """The runs kernel's contract on the decode kernel's path: an empty run writes nothing, a run longer than its
    context or than max_query_len gives NaN on the rows the call covers and leaves the rest alone, a run outside
    the rows is left alone, and a bad block id poisons only its own sequence (cut or whole)."""
    import paged_kv_cache_physical_amd as pk
    b = Batch([1400, 33, 20, 640, 9, 2100], 8, 2, 64, 16, "f32", seed=13)  # G = 4: up to 4 queries per run
    t, l = b.tables()
    runs = [3, 0, 21, 2, 9, 4]
    T = sum(runs)
    q = wl.draw_values(wl.rng_for(14, wl.STREAM_Q), (T, 8, 64), "f32")
    starts = np.concatenate([[0], np.cumsum(runs)]).astype(np.int32)
    sentinel = torch.full((T, 8, 64), 7.0, dtype=torch.float32, device="cuda")
    out, *_ = b.multi(runs, q, tables=t, lens=l, query_start=starts, max_query_len=4, out=sentinel, split=True)
    ref0 = b.oracle(q[:3], t[:1], l[:1], starts[:2])
    check_close(out[:3], ref0, "f32", "sequence 0")
    assert np.all(np.isnan(out[3:3 + 4])) and np.all(out[3 + 4:24] == 7.0)  # 21 > max_query_len and > n
    ref3 = b.oracle(q[24:26], t[3:4], l[3:4], np.array([0, 2], np.int32))
    check_close(out[24:26], ref3, "f32", "sequence 3")
    assert np.all(np.isnan(out[26:26 + 4])) and np.all(out[26 + 4:35] == 7.0)  # 9 > max_query_len
    ref5 = b.oracle(q[35:39], t[5:6], l[5:6], np.array([0, 4], np.int32))
    check_close(out[35:39], ref5, "f32", "sequence 5")
    # bad block ids in a long (cut) sequence and a short one; a run outside [0, T) is left alone
    t2 = t.copy()
    t2[0, 40] = b.nb + 5
    t2[3, 1] = b.nb + 6
    starts2 = np.array([0, 3, 3, 3, 5, T + 4, T + 6], np.int32)
    runs2 = [3, 0, 0, 2, 1, 2]
    sentinel.fill_(7.0)
    out, *_ = b.multi(runs2, q, tables=t2, lens=l, query_start=starts2, max_query_len=4, out=sentinel, split=True)
    assert np.all(np.isnan(out[:5])) and np.all(out[5:] == 7.0)
    # a workspace too small for the split is refused before any work
    assert pk.pkv_attention_multi_workspace_bytes(6, 8, 2, 64, int(l.max()), 4) > 4096
    with pytest.raises(pk.PkvError):
        pk.pkv_paged_attention_multi(sentinel, to_dev(q, "f32"), *b.caches, torch.from_numpy(t).cuda(),
                                     torch.from_numpy(l).cuda(), torch.from_numpy(starts).cuda(), int(l.max()), 4,
                                     0.125, workspace=torch.empty(4096, dtype=torch.uint8, device="cuda"))


def test_short_runs_on_the_decode_kernel_full_size_and_stable():
    """Verification of 4 drafted tokens at the Llama-7B decode shape through the decode kernel's path: every row
    against the oracle; repeated calls and graph replays give the same bits."""
    import paged_kv_cache_physical_amd as pk
    w = wl.named("llama7b_bf16", seed=0)
    s = w.spec
    runs = [4] * w.num_seqs
    lens = [int(n) for n in w.context_lens]
    b = Batch(lens, s.num_q_heads, s.num_kv_heads, s.head_dim, s.block_size, s.kv_dtype, seed=0, spare=64)
    q = wl.draw_values(wl.rng_for(17, wl.STREAM_Q), (sum(runs), s.num_q_heads, s.head_dim), s.kv_dtype)
    out, t, l, starts = b.multi(runs, q, split=True)
    check_close(out, b.oracle(q, t, l, starts), s.kv_dtype, f"all {len(runs)} runs")
    nbytes = pk.pkv_attention_multi_workspace_bytes(len(lens), s.num_q_heads, s.num_kv_heads, s.head_dim,
                                                   int(l.max()), 4)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    qd = to_dev(q, s.kv_dtype)
    bt, cl, st = torch.from_numpy(t).cuda(), torch.from_numpy(l).cuda(), torch.from_numpy(starts).cuda()
    o = torch.empty((sum(runs), s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    call = lambda: pk.pkv_paged_attention_multi(o, qd, *b.caches, bt, cl, st, int(l.max()), 4,
                                                1.0 / np.sqrt(s.head_dim), stream=stream, workspace=ws)
    with torch.cuda.stream(stream):
        call()
        torch.cuda.synchronize()
        first = o.clone()
        assert np.array_equal(first.cpu().numpy(), out)
        for i in range(3):
            o.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
            assert torch.equal(o, first), i
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            call()
        for i in range(3):
            o.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(o, first), i


SPLIT_GRID = [(dt, G, B) for dt in ("f32", "bf16") for G in (1, 4, 8) for B in (16, 32)]


@pytest.mark.parametrize("dt,G,B", SPLIT_GRID)
def test_split_context_runs(dt, G, B):
    """Few sequences with long contexts: each (sequence, KV head) is cut into context splits combined by
    log-sum-exp weights.  Lengths put runs across split boundaries, inside the first split, and past every split
    of shorter sequences; the split result matches the oracle and the unsplit call."""
    rng = wl.rng_for(300 + G + B, 1)
    lens = [2600, 1283, 770, 514, 257, 33, 1]
    runs = [min(n, int(x)) for n, x in zip(lens, rng.integers(1, 64 // G + 1, size=len(lens)))]
    Hkv = 2
    say(f"case {dt} G={G} B={B}: lens={lens} runs={runs}")
    b = Batch(lens, G * Hkv, Hkv, 128, B, dt, seed=40 + G + B)
    q = wl.draw_values(wl.rng_for(41, wl.STREAM_Q, G, B), (sum(runs), G * Hkv, 128), dt)
    out, t, l, starts = b.multi(runs, q, split=True)
    ref = b.oracle(q, t, l, starts)
    check_close(out, ref, dt, "split")
    whole, *_ = b.multi(runs, q)
    check_close(whole, ref, dt, "unsplit")
    assert np.max(np.abs(out - whole)) <= (1e-5 if dt == "f32" else 1e-3)


def test_split_context_long_verification():
    """Verification of 4 drafted tokens over 8192-token contexts (4 sequences, 32/8 heads, bf16): 32 pairs of
    (sequence, KV head), each cut into splits, against the oracle."""
    lens = [8192, 8190, 6001, 8192]
    runs = [4, 4, 4, 4]
    b = Batch(lens, 32, 8, 128, 16, "bf16", seed=51)
    q = wl.draw_values(wl.rng_for(52, wl.STREAM_Q), (16, 32, 128), "bf16")
    out, t, l, starts = b.multi(runs, q, split=True)
    check_close(out, b.oracle(q, t, l, starts), "bf16", "long verification, split")


def test_split_context_edges():
    import paged_kv_cache_physical_amd as pk
    b = Batch([1500, 900, 700], 8, 2, 64, 16, "f32", seed=61)
    t, l = b.tables()
    runs = [3, 3, 3]
    q = wl.draw_values(wl.rng_for(62, wl.STREAM_Q), (9, 8, 64), "f32")
    starts = np.array([0, 3, 6, 9], np.int32)
    nbytes = pk.pkv_attention_multi_workspace_bytes(3, 8, 2, 64, 1500, 3)
    assert nbytes > 0
    args = lambda ws: (torch.empty((9, 8, 64), dtype=torch.float32, device="cuda"), to_dev(q, "f32"), *b.caches,
                       torch.from_numpy(t).cuda(), torch.from_numpy(l).cuda(), torch.from_numpy(starts).cuda(), 1500, 3,
                       0.125)
    with pytest.raises(pk.PkvError):  # a workspace too small for the planned split
        pk.pkv_paged_attention_multi(*args(None), workspace=torch.empty(nbytes - 16, dtype=torch.uint8, device="cuda"))
    # a bad block id in the middle of sequence 0, and sequence 2 made longer than its table (its extra tokens
    # read the -1 padding): NaN rows for both, the rest exact
    t2 = t.copy()
    t2[0, 40] = b.nb + 3
    l2 = l.copy()
    l2[2] = 1501
    sentinel = torch.full((9, 8, 64), 7.0, dtype=torch.float32, device="cuda")
    out, *_ = b.multi(runs, q, tables=t2, lens=l2, out=sentinel, split=True)
    assert np.all(np.isnan(out[0:3])) and np.all(np.isnan(out[6:9]))
    ref = b.oracle(q[3:6], t[1:2], l[1:2], np.array([0, 3], np.int32))
    check_close(out[3:6], ref, "f32", "sequence 1")


def test_preemption_by_recomputation_through_the_prefix_cache():
    """Preemption by recomputation ([P4] "Preemption"): a request's blocks are freed; while it waits, other
    requests take some of them (evicting their keys); on re-admission the prompt maps what the prefix cache still
    holds, only the lost positions' K/V are written again and their rows recomputed (runs of queries), and the
    next decode step equals the oracle and the step before preemption."""
    import paged_kv_cache_physical_amd as pk
    B, Hq, Hkv, d, dt = 16, 32, 8, 128, "bf16"
    pr = wl.PrefixRequests(seed=71, num_requests=6, num_stems=2, stem_range=(300, 600), tail_range=(40, 120),
                           num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, kv_dtype=dt)
    lens = [len(pr.prompt(r)) for r in range(6)]
    nb = 67  # sized so that the waiting request's tail blocks are taken while its stem stays cached
    pool = pk.Pool(nb, B, wl.rng_for(72, wl.STREAM_PERM).permutation(nb).astype(np.int32))
    caches = pk.empty_caches(nb, Hkv, B, d, dt)
    scale = 1.0 / np.sqrt(d)

    def admit(r):
        ids = pr.prompt(r)
        sid, hit = pool.create_prefixed(ids)
        slots, pairs = pool.append([sid], [len(ids) - hit], token_ids=ids[hit:])
        assert pairs.shape == (0, 2)
        k, v = pr.kv(r)
        pk.pkv_reshape_and_cache(to_dev(k[hit:], dt), to_dev(v[hit:], dt), *caches, torch.from_numpy(slots).cuda(), B)
        return sid, hit

    def decode(sid, q):
        t, l = pool.block_tables([sid], max(-(-n // B) for n in lens))
        out = torch.empty((1, Hq, d), dtype=torch.float32, device="cuda")
        pk.pkv_paged_attention_multi(out, to_dev(q, dt), *caches, torch.from_numpy(t).cuda(), torch.from_numpy(l).cuda(),
                                     torch.tensor([0, 1], dtype=torch.int32, device="cuda"), int(l.max()), 1, scale)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    victim = 0
    sid, _ = admit(victim)
    q = wl.draw_values(wl.rng_for(73, wl.STREAM_Q), (1, Hq, d), dt)
    before = decode(sid, q)
    pool.free_seq(sid)  # preempted: its blocks wait at the tail of the free queue, still keyed
    sharer, shared = admit(2)  # request 2 has the same stem: it maps the waiting stem blocks
    assert shared == 320
    other, _ = admit(1)  # request 1 drains the queue into the victim's tail blocks, evicting their keys
    pool.free_seq(other)  # and finishes
    sid2, hit = admit(victim)  # re-admission: the stem (held by request 2) is mapped, the rest is written again
    n = lens[victim]
    assert 0 < hit < n, (hit, n)  # part of the prompt survived, part was evicted
    say(f"  re-admission mapped {hit} of {n} prompt tokens")
    # the recomputed positions' own attention rows (the prefill of what was lost), against the oracle
    t, l = pool.block_tables([sid2], max(-(-m // B) for m in lens))
    qrun = wl.draw_values(wl.rng_for(74, wl.STREAM_Q), (n - hit, Hq, d), dt)
    out = torch.empty((n - hit, Hq, d), dtype=torch.float32, device="cuda")
    pk.pkv_paged_attention_multi(out, to_dev(qrun, dt), *caches, torch.from_numpy(t).cuda(), torch.from_numpy(l).cuda(),
                                 torch.tensor([0, n - hit], dtype=torch.int32, device="cuda"), int(l.max()), n - hit, scale)
    torch.cuda.synchronize()
    k, v = (oc.to_f64(x, dt) for x in pr.kv(victim))
    ref = np.stack([oa.attention_contiguous(oc.to_f64(qrun[i], dt), k[:hit + i + 1], v[:hit + i + 1], np.float32(scale))
                    for i in range(n - hit)])
    check_close(out.cpu().numpy(), ref, dt, "recomputed rows")
    after = decode(sid2, q)
    check_close(after, oa.attention_contiguous(oc.to_f64(q[0], dt), k, v, np.float32(scale))[None], dt, "decode after")
    assert np.array_equal(after, before)  # the same tokens in other blocks: the same bits
    pool.validate()
    pool.free_seq(sharer)



@pytest.mark.parametrize("split", [False, True])
def test_sequence_order_changes_scheduling_only(split):
    """Starting the sequences longest first (or in any order) gives the same bits as the natural order; an order
    entry that is not a sequence is skipped, and the sequence it leaves out is not computed."""
    lens = [700, 2100, 33, 1500, 1, 900]
    runs = [4, 4, 4, 4, 1, 4]
    b = Batch(lens, 16, 4, 128, 16, "bf16", seed=81)
    q = wl.draw_values(wl.rng_for(82, wl.STREAM_Q), (sum(runs), 16, 128), "bf16")
    natural, t, l, starts = b.multi(runs, q, split=split)
    longest = [int(i) for i in np.argsort(-np.asarray(lens), kind="stable")]
    ordered, *_ = b.multi(runs, q, split=split, order=longest)
    assert np.array_equal(ordered, natural)
    check_close(natural, b.oracle(q, t, l, starts), "bf16", "natural order")
    sentinel = torch.full((sum(runs), 16, 128), 7.0, dtype=torch.float32, device="cuda")
    bad = [1, 3, 0, 99, 4, 2]  # sequence 5 never started; 99 skipped
    out, *_ = b.multi(runs, q, split=split, order=bad, out=sentinel)
    s5 = slice(int(starts[5]), int(starts[6]))
    if not split:  # with splits its rows are unspecified (the combine reads partials nobody wrote)
        assert np.all(out[s5] == 7.0)
    keep = np.ones(sum(runs), bool)
    keep[s5] = False
    assert np.array_equal(out[keep], natural[keep])
