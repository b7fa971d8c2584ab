"""GPU parity of preemption by swapping: pkv_swap_blocks moves blocks between the
device caches and page-locked host caches, bit for bit as the oracle's block
copy does with the oracle allocator's pairs, and attention over swapped-in
sequences gives the bits it gave before they left."""

import ctypes

import numpy as np
import pytest

import workloads as wl
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


def say(*a):
    print(*a, flush=True)


def bits(t):
    t = t.cpu() if t.is_cuda else t
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


def oracle_bits(a):
    return a.view(np.int16) if a.dtype == np.uint16 else a.view(np.int32)


@pytest.mark.parametrize("dt,B,pairs_on_host", [("bf16", 16, False), ("bf16", 32, True), ("f32", 16, True)])
def test_swap_round_trip_matches_oracle(dt, B, pairs_on_host):
    import paged_kv_cache_physical_amd as pk
    from paged_kv_cache_physical_amd.runner import GpuBatch
    w = wl.named("beam_cow_bf16", seed=2, prompts=6, beams=4, kv_dtype=dt, block_size=B, num_blocks=2048)
    s = w.spec
    host_blocks = 1024
    say(f"case {dt} B={B} pairs_on_host={pairs_on_host}: S={w.num_seqs}")
    pool = pk.Pool(w.num_blocks, B, w.free_order, host_blocks=host_blocks)
    gb = GpuBatch(w, pool=pool)
    rp = orun.replay(w, host_blocks=host_blocks)
    P = 256 if B == 16 else 512
    ref = gb.attention(P).clone()
    hk, hv = pk.empty_host_caches(host_blocks, s.num_kv_heads, B, s.head_dim, dt)
    ok, ov = oc.empty_caches(host_blocks, s.num_kv_heads, B, s.head_dim, dt)

    def move(pairs, src, dst):
        t = torch.from_numpy(pairs)
        t = t.pin_memory() if pairs_on_host else t.cuda()
        pk.pkv_swap_blocks(*src, *dst, t)
        torch.cuda.synchronize()

    # prompts 1 and 4 with their beams leave; their device blocks are free at once
    groups = [[p * s.beams + b for b in range(s.beams)] for p in (1, 4)]
    out_pairs = []
    for g in groups:
        pc, po = pool.swap_out(g), rp.pool.swap_out(g)
        assert np.array_equal(pc, po)
        move(pc, (gb.k_cache, gb.v_cache), (hk, hv))
        oc.swap_blocks(rp.k_cache, rp.v_cache, ok, ov, po)
        out_pairs.append(pc)
    hosts = np.concatenate([p[:, 1] for p in out_pairs])
    assert np.array_equal(bits(hk)[hosts], oracle_bits(ok)[hosts])
    assert np.array_equal(bits(hv)[hosts], oracle_bits(ov)[hosts])
    # another sequence takes every free device block and fills it with NaN
    x = pool.create()
    n_free = pool.stats()["free_blocks"]
    pool.append([x], [n_free * B])
    junk = torch.tensor(pool.table(x), dtype=torch.int64, device="cuda")
    gb.k_cache[junk] = float("nan")
    gb.v_cache[junk] = float("nan")
    pool.free_seq(x)
    y = rp.pool.create()
    rp.pool.append([y], [n_free * B])
    rp.pool.free_seq(y)
    # back in, groups in the other order and each group's list reversed
    for g in groups[::-1]:
        pc, po = pool.swap_in(g[::-1]), rp.pool.swap_in(g[::-1])
        assert np.array_equal(pc, po)
        move(pc, (hk, hv), (gb.k_cache, gb.v_cache))
        oc.swap_blocks(ok, ov, rp.k_cache, rp.v_cache, po)
    pool.validate()
    ids = list(range(w.num_seqs))
    tables, lens = pool.block_tables(ids, gb.max_blocks)
    ot, ol = rp.pool.block_tables(ids, gb.max_blocks)
    assert np.array_equal(tables, ot) and np.array_equal(lens, ol)
    used = np.unique(tables[tables >= 0])
    assert np.array_equal(bits(gb.k_cache)[used], oracle_bits(rp.k_cache)[used])
    assert np.array_equal(bits(gb.v_cache)[used], oracle_bits(rp.v_cache)[used])
    gb.block_tables.copy_(torch.from_numpy(tables))
    gb.out.fill_(float("nan"))
    out = gb.attention(P)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)  # the same tokens in other blocks: the same bits


def test_swap_blocks_skips_out_of_range_pairs():
    import paged_kv_cache_physical_amd as pk
    kd, vd = pk.empty_caches(4, 2, 16, 64, "f32", poison=False)
    kd.copy_(torch.randn_like(kd))
    vd.copy_(torch.randn_like(vd))
    hk, hv = pk.empty_host_caches(3, 2, 16, 64, "f32")
    hk.fill_(5.0)
    hv.fill_(5.0)
    pairs = torch.tensor([[2, 0], [4, 1], [0, 3], [1, 2]], dtype=torch.int32, device="cuda")
    pk.pkv_swap_blocks(kd, vd, hk, hv, pairs)
    torch.cuda.synchronize()
    assert torch.equal(hk[0], kd[2].cpu()) and torch.equal(hv[0], vd[2].cpu())
    assert torch.equal(hk[2], kd[1].cpu()) and torch.equal(hv[2], vd[1].cpu())
    assert bool((hk[1] == 5.0).all()) and bool((hv[1] == 5.0).all())  # source id 4 is out of range


def test_swap_blocks_refuses_memory_the_gpu_cannot_reach(libpkv):
    import paged_kv_cache_physical_amd as pk
    from paged_kv_cache_physical_amd import _lib
    kd, vd = pk.empty_caches(4, 2, 16, 64, "f32", poison=False)
    hk, hv = pk.empty_host_caches(4, 2, 16, 64, "f32")
    pairs = torch.tensor([[0, 0]], dtype=torch.int32, device="cuda")
    plain = torch.zeros_like(hk)  # pageable host memory
    assert not plain.is_pinned()
    with pytest.raises(pk.InvalidArg):
        pk.pkv_swap_blocks(kd, vd, plain, hv, pairs)
    # The library checks too: each call below must be refused before any launch.  The pairs are chosen
    # so that a launch, were a check to let one through, would still touch nothing outside real
    # allocations: the pageable case names only ids the kernel skips, the range cases only block 0.
    bb = kd[0].numel() * 4
    vp = ctypes.c_void_p
    skipped = torch.tensor([[9, 9]], dtype=torch.int32, device="cuda")

    def call(sk, dk, nsrc, ndst, pr):
        return libpkv.pkv_swap_blocks(vp(sk.data_ptr()), vp(vd.data_ptr()), vp(dk.data_ptr()), vp(hv.data_ptr()),
                                      vp(pr.data_ptr()), 1, nsrc, ndst, bb, None)

    assert call(kd, plain, 4, 4, skipped) == _lib.PKV_ERR_INVALID_ARG  # pageable destination
    assert call(kd, hk, 4, 4096, pairs) == _lib.PKV_ERR_INVALID_ARG  # past the host allocation
    assert call(kd, hk, 1 << 20, 4, pairs) == _lib.PKV_ERR_INVALID_ARG  # past the device allocation
    torch.cuda.synchronize()


DEBUG_CHILD = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
import paged_kv_cache_physical_amd as pk
kc, vc = pk.empty_caches(8, 2, 16, 64, "bf16")
k = torch.randn(3, 2, 64, device="cuda").to(torch.bfloat16)
v = torch.randn(3, 2, 64, device="cuda").to(torch.bfloat16)
def refused(fn):
    try:
        fn()
    except pk.InvalidArg:
        return True
    return False
# two writers of slot 5 are refused; a skipped (-1) or out-of-range slot may repeat
assert refused(lambda: pk.pkv_reshape_and_cache(k, v, kc, vc, torch.tensor([5, 7, 5], device="cuda"), 16))
pk.pkv_reshape_and_cache(k, v, kc, vc, torch.tensor([5, -1, -1], device="cuda"), 16)
pk.pkv_reshape_and_cache(k, v, kc, vc, torch.tensor([1, 999, 999], device="cuda"), 16)
torch.cuda.synchronize()
assert torch.equal(kc.view(8, 2, 8, 16, 8)[0, :, :, 5, :].reshape(2, 64), k[0])
# two copies into block 3 are refused; distinct targets pass
assert refused(lambda: pk.pkv_copy_blocks(kc, vc, torch.tensor([[0, 3], [1, 3]], dtype=torch.int32, device="cuda")))
pk.pkv_copy_blocks(kc, vc, torch.tensor([[0, 3], [1, 4], [9, 4]], dtype=torch.int32, device="cuda"))
torch.cuda.synchronize()
assert torch.equal(kc[3].view(torch.int16), kc[0].view(torch.int16))
print("debug checks ok", flush=True)
"""


def test_debug_mode_refuses_duplicate_write_targets():
    """With PKV_DEBUG set, reshape_and_cache and copy_blocks refuse two writers of one slot / block before
    launching (a child process: the setting is read once per process)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PKV_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", DEBUG_CHILD, root], capture_output=True, text=True, timeout=240, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "debug checks ok" in r.stdout
