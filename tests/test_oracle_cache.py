"""Pins for the oracle's cache layout, scatter, block copy and gather: byte offsets
stated by the interface's layout definition, a brute-force slot dictionary, and
round trips."""

import numpy as np
import pytest

import workloads as wl
from oracle import cache as oc


@pytest.mark.parametrize("kv_dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_layout_offsets(kv_dtype, d):
    # Interface definition: K[nb][H][d/X][B][X] with X = 16 bytes / scalar size; V[nb][H][d][B].
    nb, H, B = 5, 3, 16
    k, v = oc.empty_caches(nb, H, B, d, kv_dtype)
    item = 4 if kv_dtype == "f32" else 2
    X = 16 // item
    rng = np.random.default_rng(0)
    kt = wl.draw_values(rng, (1, H, d), kv_dtype)
    vt = wl.draw_values(rng, (1, H, d), kv_dtype)
    blk, off = 3, 11
    oc.scatter(k, v, kt, vt, np.array([blk * B + off]))
    kf = k.reshape(-1)
    vf = v.reshape(-1)
    for h in range(H):
        for e in range(d):
            kidx = (((blk * H + h) * (d // X) + e // X) * B + off) * X + e % X
            vidx = ((blk * H + h) * d + e) * B + off
            assert kf[kidx].tobytes() == kt[0, h, e].tobytes()
            assert vf[vidx].tobytes() == vt[0, h, e].tobytes()
    # everything else is still poison
    poison = oc.POISON[kv_dtype]
    written_k = np.zeros(kf.size, bool)
    for h in range(H):
        for e in range(d):
            written_k[(((blk * H + h) * (d // X) + e // X) * B + off) * X + e % X] = True
    assert np.all(kf.view(poison.dtype)[~written_k] == poison)
    written_v = np.zeros(vf.size, bool)
    for h in range(H):
        for e in range(d):
            written_v[((blk * H + h) * d + e) * B + off] = True
    assert np.all(vf.view(poison.dtype)[~written_v] == poison)


def test_scatter_gather_against_slot_dictionary():
    rng = np.random.default_rng(5)
    nb, H, B, d = 12, 2, 16, 64
    for kv_dtype in ("f32", "bf16"):
        k, v = oc.empty_caches(nb, H, B, d, kv_dtype)
        truth = {}
        for _ in range(4):
            slots = rng.choice(nb * B, size=20, replace=False).astype(np.int64)
            slots[rng.integers(0, 20)] = -1  # skipped
            kt = wl.draw_values(rng, (20, H, d), kv_dtype)
            vt = wl.draw_values(rng, (20, H, d), kv_dtype)
            oc.scatter(k, v, kt, vt, slots)
            for i, s in enumerate(slots):
                if s >= 0:
                    truth[int(s)] = (kt[i].copy(), vt[i].copy())
        # read every slot back through a one-block-per-entry table
        for s, (kt, vt) in truth.items():
            table = [s // B]
            kg, vg = oc.gather(k, v, table, s % B + 1)
            assert kg[s % B].tobytes() == kt.tobytes()
            assert vg[s % B].tobytes() == vt.tobytes()


def test_gather_reassembles_logical_order():
    rng = np.random.default_rng(9)
    nb, H, B, d = 10, 2, 16, 128
    k, v = oc.empty_caches(nb, H, B, d, "bf16")
    n = 37
    table = [7, 2, 5]
    kt = wl.draw_values(rng, (n, H, d), "bf16")
    vt = wl.draw_values(rng, (n, H, d), "bf16")
    slots = np.array([table[t // B] * B + t % B for t in range(n)])
    oc.scatter(k, v, kt, vt, slots)
    kg, vg = oc.gather(k, v, table, n)
    assert np.array_equal(kg, kt) and np.array_equal(vg, vt)


def test_copy_blocks_sequential_semantics():
    rng = np.random.default_rng(1)
    nb, H, B, d = 6, 2, 16, 64
    k, v = oc.empty_caches(nb, H, B, d, "f32")
    k[...] = rng.standard_normal(k.shape, dtype=np.float32)
    v[...] = rng.standard_normal(v.shape, dtype=np.float32)
    k0, v0 = k.copy(), v.copy()
    oc.copy_blocks(k, v, np.array([[1, 4], [3, 0]], np.int32))
    assert np.array_equal(k[4], k0[1]) and np.array_equal(v[4], v0[1])
    assert np.array_equal(k[0], k0[3]) and np.array_equal(v[0], v0[3])
    for b in (1, 2, 3, 5):
        assert np.array_equal(k[b], k0[b]) and np.array_equal(v[b], v0[b])


def test_scatter_rejects_bad_slots():
    k, v = oc.empty_caches(2, 1, 16, 64, "f32")
    x = np.zeros((2, 1, 64), np.float32)
    with pytest.raises(ValueError):
        oc.scatter(k, v, x, x, np.array([3, 3]))
    with pytest.raises(ValueError):
        oc.scatter(k, v, x, x, np.array([0, 32]))


def test_bf16_widening_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-3], np.float32)
    b = wl.f32_to_bf16_bits(x)
    y = oc.to_f64(b, "bf16")
    # bf16 keeps 8 significant bits: these are representable exactly except 1e-3
    assert y[0] == 1.0 and y[1] == -2.5 and y[2] == 3.140625
    assert abs(y[3] - 1e-3) <= 2 ** -9 * 1e-3 * 2
    # round-to-nearest-even at a tie: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1 (even)
    t = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32)
    assert list(oc.to_f64(wl.f32_to_bf16_bits(t), "bf16")) == [1.0, 1 + 2 ** -6]
