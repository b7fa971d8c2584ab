"""GPU parity of automatic prefix caching: requests that share prompt stems are
admitted through pkv_seq_create_prefixed, only their uncached tokens are
written (pkv_reshape_and_cache at the slots pkv_append_tokens returns), and
attention over the resulting tables equals the float64 oracle computed from
each request's own contiguous K/V; the same requests built without prefix
caching (every token written to a private block) give the same bits."""

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
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits(t):
    t = t.cpu()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


def attention(pk, caches, tables, lens, q_dev, B, P):
    S, Hq, d = q_dev.shape
    max_n = int(lens.max())
    ws_bytes = pk.pkv_attention_workspace_bytes(S, Hq, caches[1].shape[1], d, B, max_n, P)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.full((S, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    pk.pkv_paged_attention_decode(out, q_dev, caches[0], caches[1], torch.from_numpy(tables).cuda(),
                                  torch.from_numpy(lens).cuda(), max_n, 1.0 / np.sqrt(d), P, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dt,B", [("bf16", 16), ("bf16", 32), ("f32", 16)])
def test_prefix_cached_requests_match_oracle(dt, B):
    import paged_kv_cache_physical_amd as pk
    R, Hq, Hkv, d = 48, 32, 8, 128
    pr = wl.PrefixRequests(seed=11 + B, num_requests=R, num_stems=4, stem_range=(200, 1100), tail_range=(1, 300),
                           num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, kv_dtype=dt)
    lens_all = [len(pr.prompt(r)) for r in range(R)]
    nb = sum(-(-n // B) for n in lens_all) + 64
    order = wl.rng_for(3, wl.STREAM_PERM).permutation(nb).astype(np.int32)
    say(f"case {dt} B={B}: R={R} blocks={nb} max_n={max(lens_all)}")
    pool, opool = pk.Pool(nb, B, order), al.BlockPool(nb, B, order)
    caches = pk.empty_caches(nb, Hkv, B, d, dt)
    ocaches = oc.empty_caches(nb, Hkv, B, d, dt)

    def admit(r):
        ids = pr.prompt(r)
        (sid, hit), (osid, ohit) = pool.create_prefixed(ids), opool.create_prefixed(ids)
        assert (sid, hit) == (osid, ohit)
        slots, pairs = pool.append([sid], [len(ids) - hit], token_ids=ids[hit:])
        oslots, opairs = opool.append([osid], [len(ids) - ohit], token_ids=ids[ohit:])
        assert np.array_equal(slots, oslots) and pairs.shape == (0, 2) and opairs.shape == (0, 2)
        k, v = pr.kv(r)
        pk.pkv_reshape_and_cache(to_dev(k[hit:], dt), to_dev(v[hit:], dt), caches[0], caches[1],
                                 torch.from_numpy(slots).cuda(), B)
        oc.scatter(ocaches[0], ocaches[1], k[hit:], v[hit:], oslots)
        return sid, hit

    # first wave: the first request of each stem computes it, the others find it
    seqs, hits = {}, 0
    for r in range(R // 2):
        seqs[r], h = admit(r)
        hits += h
    # some requests finish: their stem blocks wait in the free queue, still findable
    for r in range(0, R // 2, 3):
        pool.free_seq(seqs[r])
        opool.free_seq(seqs.pop(r))
    st = pool.stats()
    assert st == opool.stats() and st["cached_free_blocks"] > 0
    for r in range(R // 2, R):
        seqs[r], h = admit(r)
        hits += h
    pool.validate()
    assert pool.cached() == opool.cached
    assert hits > R * 150, hits  # most stem tokens were mapped, not written
    say(f"  mapped {hits} prompt tokens of {sum(lens_all)} from the prefix cache")
    live = sorted(seqs)
    ids = [seqs[r] for r in live]
    max_blocks = max(-(-lens_all[r] // B) for r in live)
    tables, lens = pool.block_tables(ids, max_blocks)
    ot, ol = opool.block_tables(ids, max_blocks)
    assert np.array_equal(tables, ot) and np.array_equal(lens, ol)
    used = np.unique(tables[tables >= 0])
    assert np.array_equal(bits(caches[0])[used], ocaches[0].view(np.int16 if dt == "bf16" else np.int32)[used])
    assert np.array_equal(bits(caches[1])[used], ocaches[1].view(np.int16 if dt == "bf16" else np.int32)[used])

    q = pr.q()[live]
    q_dev = to_dev(q, dt)
    ref = np.stack([oa.attention_contiguous(oc.to_f64(q[i], dt), *(oc.to_f64(x, dt) for x in pr.kv(r)),
                                            1.0 / np.sqrt(d)) for i, r in enumerate(live)])
    outs = {}
    for P in (0, 256):
        out = attention(pk, caches, tables, lens, q_dev, B, P).cpu().numpy()
        assert np.all(np.isfinite(out))
        err = float(np.max(np.abs(out - ref)))
        rl2 = float(np.linalg.norm(out - ref) / np.linalg.norm(ref))
        say(f"  P={P}: max_abs={err:.3e} rel_l2={rl2:.3e}")
        assert (err <= 1e-5) if dt == "f32" else (err <= 1e-2 and rl2 <= 2e-3)
        assert rl2 <= 1e-4
        outs[P] = out

    # the same requests with private blocks: every token written, no key ever looked up
    priv = pk.Pool(nb * 2, B)
    pcaches = pk.empty_caches(nb * 2, Hkv, B, d, dt)
    pids = []
    for r in live:
        sid = priv.create()
        slots, _ = priv.append([sid], [lens_all[r]])
        k, v = pr.kv(r)
        pk.pkv_reshape_and_cache(to_dev(k, dt), to_dev(v, dt), pcaches[0], pcaches[1],
                                 torch.from_numpy(slots).cuda(), B)
        pids.append(sid)
    assert priv.stats()["cached_blocks"] == 0
    ptables, plens = priv.block_tables(pids, max_blocks)
    assert np.array_equal(plens, lens)
    for P in (0, 256):
        out = attention(pk, pcaches, ptables, plens, q_dev, B, P).cpu().numpy()
        assert np.array_equal(out, outs[P])  # the same tokens in other blocks: the same bits
