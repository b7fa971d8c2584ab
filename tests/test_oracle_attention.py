"""Pins for the oracle's float64 attention: an independent library routine (torch's
scaled_dot_product_attention on the CPU in float64), closed-form special cases,
and the invariants the pages imply (paging changes storage, not results)."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as oa
from oracle import cache as oc
from oracle import run as orun


def rand(rng, *shape):
    return rng.standard_normal(shape)


def sdpa_reference(q, k, v, scale):
    """torch SDPA (float64, CPU) with KV heads repeated per query group."""
    Hq = q.shape[0]
    Hkv = k.shape[1]
    G = Hq // Hkv
    Q = torch.from_numpy(q)[:, None, :]  # [Hq][1][d]
    K = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq][n][d]
    V = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=float(scale))
    return out[:, 0, :].numpy()


@pytest.mark.parametrize("Hq,Hkv,n,d", [(8, 8, 37, 64), (8, 2, 1, 16), (64, 8, 300, 128), (4, 1, 17, 32),
                                        (2, 2, 1000, 8)])
def test_matches_torch_sdpa(Hq, Hkv, n, d):
    rng = np.random.default_rng(Hq * 1000 + n)
    q, k, v = rand(rng, Hq, d), rand(rng, n, Hkv, d), rand(rng, n, Hkv, d)
    scale = np.float32(1 / np.sqrt(d))
    ref = sdpa_reference(q, k, v, scale)
    out = oa.attention_contiguous(q, k, v, scale)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_single_token_returns_value_exactly():
    rng = np.random.default_rng(0)
    q, k, v = rand(rng, 4, 8), rand(rng, 1, 2, 8), rand(rng, 1, 2, 8)
    out = oa.attention_contiguous(q, k, v, 0.3)
    assert np.array_equal(out[:2], np.repeat(v[0, :1], 2, axis=0))
    assert np.array_equal(out[2:], np.repeat(v[0, 1:], 2, axis=0))


def test_zero_query_is_mean_of_values():
    rng = np.random.default_rng(1)
    k, v = rand(rng, 50, 2, 8), rand(rng, 50, 2, 8)
    out = oa.attention_contiguous(np.zeros((2, 8)), k, v, 0.5)
    assert np.allclose(out, v.mean(axis=0), atol=1e-14, rtol=0)


def test_equal_keys_is_mean_of_values():
    rng = np.random.default_rng(2)
    k = np.repeat(rand(rng, 1, 1, 16), 33, axis=0)
    v = rand(rng, 33, 1, 16)
    out = oa.attention_contiguous(rand(rng, 1, 16), k, v, 0.25)
    assert np.allclose(out[0], v[:, 0].mean(axis=0), atol=1e-14, rtol=0)


def test_constant_values_pass_through():
    rng = np.random.default_rng(3)
    c = rand(rng, 16)
    v = np.broadcast_to(c, (40, 1, 16)).copy()
    out = oa.attention_contiguous(rand(rng, 1, 16), rand(rng, 40, 1, 16), v, 0.25)
    assert np.allclose(out[0], c, atol=1e-14, rtol=0)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(4)
    d = 16
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    k = rand(rng, 64, 1, d) * 0.01
    j = 41
    k[j, 0, 0] = 40.0  # score 40 * scale(=1) vs ~0.01 for the rest -> weight ~ 1 - 63 e^-40
    v = rand(rng, 64, 1, d)
    out = oa.attention_contiguous(q, k, v, 1.0)
    assert np.allclose(out[0], v[j, 0], atol=1e-14, rtol=0)


def test_negative_dominant_key_is_ignored():
    # a key scoring -inf-like (far below the rest) contributes nothing: same as dropping it
    rng = np.random.default_rng(5)
    d = 8
    q = np.ones((1, d))
    k, v = rand(rng, 20, 1, d), rand(rng, 20, 1, d)
    k2 = k.copy()
    k2[7, 0, :] = -1e3
    a = oa.attention_contiguous(q, k2, v, 1.0)
    b = oa.attention_contiguous(q, np.delete(k, 7, axis=0), np.delete(v, 7, axis=0), 1.0)
    assert np.allclose(a, b, atol=1e-14, rtol=0)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(6)
    Hq, Hkv, n, d = 8, 2, 29, 16
    q, k, v = rand(rng, Hq, d), rand(rng, n, Hkv, d), rand(rng, n, Hkv, d)
    G = Hq // Hkv
    a = oa.attention_contiguous(q, k, v, 0.25)
    b = oa.attention_contiguous(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.25)
    assert np.array_equal(a, b)


def test_scale_and_query_trade_off():
    rng = np.random.default_rng(7)
    q, k, v = rand(rng, 2, 8), rand(rng, 30, 2, 8), rand(rng, 30, 2, 8)
    a = oa.attention_contiguous(q, k, v, 0.5)
    b = oa.attention_contiguous(q * 4.0, k, v, 0.125)
    assert np.allclose(a, b, atol=1e-13, rtol=0)


def test_linear_in_values_and_token_order_free():
    rng = np.random.default_rng(8)
    q, k = rand(rng, 2, 8), rand(rng, 30, 1, 8)
    v1, v2 = rand(rng, 30, 1, 8), rand(rng, 30, 1, 8)
    a = oa.attention_contiguous(q, k, v1 + 2 * v2, 0.3)
    b = oa.attention_contiguous(q, k, v1, 0.3) + 2 * oa.attention_contiguous(q, k, v2, 0.3)
    assert np.allclose(a, b, atol=1e-13, rtol=0)
    perm = rng.permutation(30)
    c = oa.attention_contiguous(q, k[perm], v1[perm], 0.3)
    assert np.allclose(c, oa.attention_contiguous(q, k, v1, 0.3), atol=1e-14, rtol=0)


@pytest.mark.parametrize("P", [1, 16, 37, 64, 512, 10_000])
def test_split_context_equals_direct(P):
    rng = np.random.default_rng(P)
    q, k, v = rand(rng, 8, 16), rand(rng, 700, 2, 16), rand(rng, 700, 2, 16)
    a = oa.attention_contiguous(q, k, v, 0.25)
    b = oa.attention_split(q, k, v, 0.25, P)
    assert np.max(np.abs(a - b)) < 1e-12


def _paged_out(w, seed_order=None):
    if seed_order is not None:
        w.free_order = np.random.default_rng(seed_order).permutation(w.num_blocks).astype(np.int32)
    rp = orun.replay(w)
    s = w.spec
    return rp, oa.paged_attention(w.q, rp.k_cache, rp.v_cache, rp.tables, rp.context_lens, w.scale, s.kv_dtype)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_paged_equals_contiguous_and_ignores_placement(kv_dtype):
    w = wl.small_decode(6, (1, 90), 8, 2, 64, 16, kv_dtype, seed=11)
    rp, out = _paged_out(w)
    # contiguous baseline from the generator's logical tokens
    for s in range(w.num_seqs):
        k, v = w.token_kv(s)
        ref = oa.attention_contiguous(oc.to_f64(w.q[s], kv_dtype), oc.to_f64(k, kv_dtype), oc.to_f64(v, kv_dtype),
                                      w.scale)
        assert np.array_equal(out[s], ref)
    # the unused slots are NaN-poisoned, yet nothing NaN reaches the output
    assert np.all(np.isfinite(out))
    # any other placement of the physical blocks gives bit-identical output
    w2 = wl.small_decode(6, (1, 90), 8, 2, 64, 16, kv_dtype, seed=11)
    rp2, out2 = _paged_out(w2, seed_order=99)
    assert not np.array_equal(rp.tables, rp2.tables)
    assert np.array_equal(out, out2)


def test_shared_prefix_equals_private_copies():
    w = wl.named("beam_cow_bf16", seed=3, prompts=2, prefix_len=40, tail_range=(1, 20), num_blocks=64)
    rp = orun.replay(w)
    out = oa.paged_attention(w.q, rp.k_cache, rp.v_cache, rp.tables, rp.context_lens, w.scale, "bf16")
    # beams really share physical blocks
    assert rp.tables[0, 0] == rp.tables[1, 0] == rp.tables[3, 0]
    for s in range(w.num_seqs):
        k, v = w.token_kv(s)  # private, contiguous copy of the beam's tokens
        ref = oa.attention_contiguous(oc.to_f64(w.q[s], "bf16"), oc.to_f64(k, "bf16"), oc.to_f64(v, "bf16"), w.scale)
        assert np.array_equal(out[s], ref)
