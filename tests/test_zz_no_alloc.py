"""pkv_decode_step_static, the decode step for callers that cannot allocate: it takes the split-context
workspace from the library's static device scratch instead of a caller argument.  Its kernels are those of
pkv_decode_step, so the output and the caches must equal that entry point's bit for bit; two calls in a row,
the second with a smaller batch of another shape (the scratch keeps the first call's contents)."""

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oa
from oracle import run as orun

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu(libpkv):
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    yield
    torch.cuda.synchronize()


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).clone()


def test_static_scratch_step_equals_workspace_step():
    import paged_kv_cache_physical_amd as pk
    from paged_kv_cache_physical_amd.runner import GpuBatch
    cases = [
        # the full-size GQA batch (256 sequences, 64/8 heads, lognormal lengths), then a smaller batch of another
        # shape (40 sequences, 16/4 heads, d 64, B 32)
        (wl.named("gqa_bf16_b16", seed=0), 512),
        (wl.small_decode(40, (100, 3000), 16, 4, 64, 32, "bf16", seed=3), 64),
    ]
    for w, P in cases:
        s = w.spec
        print(f"case {s.name}: S={w.num_seqs} Hq={s.num_q_heads} Hkv={s.num_kv_heads} d={s.head_dim} "
              f"B={s.block_size} P={P}", flush=True)
        assert pk.pkv_attention_workspace_bytes(w.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                                s.block_size, w.max_context_len, P) > 0
        gb = GpuBatch(w)
        ref = gb.step(P).clone()
        k0, v0 = bits(gb.k_cache), bits(gb.v_cache)
        for rep in range(2):
            out = torch.full_like(gb.out, float("nan"))
            d = gb.decode
            pk.pkv_decode_step_static(d.k_new, d.v_new, out, gb.q, gb.k_cache, gb.v_cache, gb.block_tables,
                                      gb.context_lens, gb.max_context_len, float(w.scale), P)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), (s.name, rep)
            assert torch.equal(bits(gb.k_cache), k0) and torch.equal(bits(gb.v_cache), v0)
        if w.num_seqs <= 64:
            rp = orun.replay(w)
            exp = oa.paged_attention(w.q, rp.k_cache, rp.v_cache, rp.tables, rp.context_lens, w.scale, s.kv_dtype)
            got = out.cpu().numpy()
            err = float(np.max(np.abs(got - exp)))
            rl2 = float(np.linalg.norm(got - exp) / np.linalg.norm(exp))
            print(f"  against the oracle: max_abs={err:.3e} rel_l2={rl2:.3e}", flush=True)
            assert err <= 1e-2 and rl2 <= 1e-4
        del gb
