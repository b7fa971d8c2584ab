#!/usr/bin/env python3
"""Benchmark of the paged decode-attention step on one MI355X.

A step is one pass of the decode hot path over a synthetic batch already
resident in HBM: write each sequence's new K/V token into its slot, then
paged decode attention over every context, with the log-sum-exp combination
of contexts cut between workgroups.  The step is one pkv_decode_step call, one
kernel launch for up to 4096 sequences: the kernel writes the new tokens in
its set-up and combines cut sequences at the end.  The same step as two calls
(reshape_and_cache, then attention) and the two-stage attention (partition
pass, then a separate combination) are timed beside it.  The block pool,
tables and the rest of the context are built once before timing by the
library's own allocator and kernels.

Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-extra] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak, 8 TB/s
METRIC = "decode-attention KV GB/s (% of HBM peak) and seq-steps/sec at 1 MI355X"
# The headline: the largest single-GPU decode batch (256 sequences, GQA 64/8 heads, lognormal contexts).
HEADLINE = "gqa_bf16_b16"
EXTRA = ["llama7b_bf16", "gqa_bf16_b32", "long_bf16", "beam_cow_bf16"]
_CSRC = os.path.join(ROOT, "paged_kv_cache_physical_amd", "csrc")
# Source files of each kernel family; a profile-derived number is used only while its family's hash matches.
KERNEL_FAMILIES = {
    "decode": ("attention.hip", "device_common.h"),
    "multi_query": ("multi_query.hip", "device_common.h"),
    "cache_ops": ("cache_ops.hip", "device_common.h"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """Source text without comments and blank lines: edits to comments keep the hash."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in src.splitlines())
    return "\n".join(line for line in lines if line.strip())


def kernel_sha(family: str = "decode") -> str:
    """Hash of one kernel family's code (ties profile-derived numbers to the code they measured)."""
    h = hashlib.sha256()
    for name in KERNEL_FAMILIES[family]:
        with open(os.path.join(_CSRC, name), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def source_shas() -> dict:
    return {fam: kernel_sha(fam) for fam in KERNEL_FAMILIES}


def describe(w) -> dict:
    s = w.spec
    d = {"workload": s.name, "num_seqs": w.num_seqs, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
         "head_dim": s.head_dim, "block_size": s.block_size, "kv_dtype": s.kv_dtype,
         "partition_size": s.partition_size, "total_context_tokens": w.total_tokens,
         "max_context_len": w.max_context_len, "pool_blocks": w.num_blocks, "seed": s.seed,
         "kv_bytes_per_step": w.kv_bytes}
    if s.kind == "beam":
        d["lengths"] = f"{s.prefix_len} shared + uniform{list(s.tail_range)}"
    elif s.lens is not None:
        d["lengths"] = list(s.lens)
    else:
        d["lengths"] = str(s.len_dist)
    return d


def time_launches(fn, n, stream):
    """Average duration (ms) of n launches of fn, each bracketed by HIP events on `stream`."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return float(t.mean()), float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def unique_kv_bytes(w, tables, lens) -> int:
    """Bytes of the distinct physical slots the step reads (shared prefix blocks counted once)."""
    B = w.spec.block_size
    slots = set()
    for t, n in zip(tables, lens):
        for pos in range(int(n)):
            slots.add(int(t[pos // B]) * B + pos % B)
    return len(slots) * w.kv_bytes_per_token


def measure(w, steps, warmup, stream):
    import torch
    from paged_kv_cache_physical_amd.runner import GpuBatch

    t0 = time.perf_counter()
    gb = GpuBatch(w)
    log(f"[bench] {w.spec.name}: built batch ({w.total_tokens} tokens, {w.kv_bytes / 1e9:.3f} GB KV) "
        f"in {time.perf_counter() - t0:.1f}s")
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            gb.step(stream=stream)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        start.record(stream)
        for _ in range(steps):
            gb.step(stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms_step = start.elapsed_time(end) / steps
        n_k = max(steps, 20)
        part = time_launches(lambda: gb.attention_partitions(stream=stream), n_k, stream)
        red = time_launches(lambda: gb.attention_reduce(stream=stream), n_k, stream)
        rc = time_launches(lambda: gb.write_decode_token(stream=stream), n_k, stream)
        attn = time_launches(lambda: gb.attention(stream=stream), n_k, stream)
        sep = time_launches(lambda: gb.step_separate(stream=stream), n_k, stream)
        stp = time_launches(lambda: gb.step(stream=stream), n_k, stream)  # per-step spread
    res = {
        "ms_per_step": ms_step,
        "wall_ms_per_step": 1e3 * wall / steps,
        "kv_gbps_step": w.kv_bytes / (ms_step * 1e-3) / 1e9,
        "seq_steps_per_s": w.num_seqs / (ms_step * 1e-3),
        "partition_kernel_us": {"mean": 1e3 * part[0], "median": 1e3 * part[1], "p10": 1e3 * part[2],
                                "p90": 1e3 * part[3]},
        "step_us": {"mean": 1e3 * stp[0], "median": 1e3 * stp[1], "p10": 1e3 * stp[2], "p90": 1e3 * stp[3]},
        "reduce_kernel_us": 1e3 * red[0],
        "reshape_and_cache_us": 1e3 * rc[0],
        "attention_us": 1e3 * attn[0],
        "separate_calls_step_us": 1e3 * sep[0],
        "kv_gbps_partition_kernel": w.kv_bytes / (part[0] * 1e-3) / 1e9,
        "kv_gbps_attention": w.kv_bytes / (attn[0] * 1e-3) / 1e9,
        "kv_gbps_step_launch": w.kv_bytes / (stp[0] * 1e-3) / 1e9,
    }
    pairs = [p for p in gb.pairs if len(p)]
    if pairs:  # copy-on-write copies made while building the batch, re-issued: idempotent
        pd = torch.from_numpy(np.concatenate(pairs)).to("cuda")
        from paged_kv_cache_physical_amd import pkv_copy_blocks
        with torch.cuda.stream(stream):
            cb = time_launches(lambda: pkv_copy_blocks(gb.k_cache, gb.v_cache, pd, stream), n_k, stream)
        res["copy_blocks_pairs"] = int(pd.shape[0])
        res["copy_blocks_us"] = 1e3 * cb[0]
    if w.spec.kind == "beam":  # shared prefixes: logical bytes count them per sequence, unique bytes once
        ub = unique_kv_bytes(w, gb.tables_host, gb.lens_host)
        res["unique_kv_bytes"] = ub
        res["unique_kv_gbps_partition_kernel"] = ub / (part[0] * 1e-3) / 1e9
    del gb
    torch.cuda.empty_cache()
    return res


def host_allocator_step_us(w, reps=20):
    """Host side of a decode step (append one token to every sequence, then refresh the block tables
    and lengths), timed on a host-only replay of the batch's allocator script."""
    from paged_kv_cache_physical_amd import Pool
    from workloads import Append, Create, Fork
    pool = Pool(w.num_blocks, w.spec.block_size, w.free_order)
    ids = []
    for op in w.script():
        if isinstance(op, Create):
            ids.extend(pool.create() for _ in range(op.count))
        elif isinstance(op, Fork):
            ids.append(pool.fork(op.parent))
        elif isinstance(op, Append):
            pool.append(op.seqs, op.counts)
    seqs = np.asarray(sorted(ids), dtype=np.int32)
    ones = np.ones(len(seqs), dtype=np.int32)
    # table width sized once, with room for the appended tokens (a server keeps a fixed-width table)
    mb = max(pool.info(int(i))[1] for i in seqs) + 2 * reps // w.spec.block_size + 2
    t = []
    for _ in range(reps):
        t0 = time.perf_counter()
        pool.append(seqs, ones)
        pool.block_tables(seqs, mb)
        t.append(time.perf_counter() - t0)
    # the same two C calls with buffers allocated once, as a native serving loop makes them
    import ctypes
    from paged_kv_cache_physical_amd import _lib
    L = _lib.lib()
    n = len(seqs)
    slots = np.empty(n, np.int64)
    pairs = np.empty((n, 2), np.int32)
    tables = np.empty((n, mb + reps // w.spec.block_size + 1), np.int32)
    lens = np.empty(n, np.int32)
    ncow = ctypes.c_int32()
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    ps, po, pslot, ppair, ptab, plen = P(seqs), P(ones), P(slots), P(pairs), P(tables), P(lens)
    tc = []
    for _ in range(reps):
        t0 = time.perf_counter()
        L.pkv_append_tokens(pool.handle, ps, po, n, None, pslot, n, ppair, n, ctypes.byref(ncow))
        L.pkv_block_tables(pool.handle, ps, n, tables.shape[1], ptab, plen)
        tc.append(time.perf_counter() - t0)
    return 1e6 * float(np.median(t)), 1e6 * float(np.median(tc))


def measure_prefix_cache(requests=256, stems=8, block_size=16):
    """Automatic prefix caching on the host pool: requests over a few shared stems (1000-2000 tokens, as a
    system prompt or few-shot header) with their own tails (1-256 tokens) are admitted one by one
    (pkv_seq_create_prefixed, then pkv_append_tokens of the uncached ids).  Reports the host time per admitted
    request, the prompt tokens mapped from the cache instead of written, and the blocks in use against the same
    requests with private blocks."""
    import workloads as wl
    from paged_kv_cache_physical_amd import Pool
    pr = wl.PrefixRequests(seed=0, num_requests=requests, num_stems=stems, stem_range=(1000, 2000),
                           tail_range=(1, 256), num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype="bf16")
    prompts = [np.asarray(pr.prompt(r), dtype=np.int32) for r in range(requests)]  # ids as the binding takes them
    need = sum(-(-len(p) // block_size) for p in prompts)
    pool = Pool(need, block_size, np.random.default_rng(0).permutation(need).astype(np.int32))
    mapped, t = 0, []
    for ids in prompts:
        t0 = time.perf_counter()
        sid, hit = pool.create_prefixed(ids)
        pool.append([sid], [len(ids) - hit], token_ids=ids[hit:])
        t.append(time.perf_counter() - t0)
        mapped += hit
    st = pool.stats()
    total = sum(len(p) for p in prompts)
    return {"requests": requests, "stems": stems, "prompt_tokens": total, "tokens_from_cache": mapped,
            "fraction_from_cache": round(mapped / total, 4), "blocks_used": st["used_blocks"],
            "blocks_private": need, "cached_blocks": st["cached_blocks"],
            "host_us_per_request_median": round(1e6 * float(np.median(t)), 2),
            "host_us_per_request_mean": round(1e6 * float(np.mean(t)), 2)}


def hbm_read_ceiling(stream):
    """Practical HBM read rate of a plain streaming kernel over 4 GiB (context for the roofline)."""
    import torch
    from paged_kv_cache_physical_amd import pkv_hbm_read_probe
    x = torch.ones(4 * 1024 ** 3 // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(3):
            pkv_hbm_read_probe(x, sink, stream)
        ms = time_launches(lambda: pkv_hbm_read_probe(x, sink, stream), 20, stream)[1]
    del x
    torch.cuda.empty_cache()
    return 4 * 1024 ** 3 / (ms * 1e-3) / 1e9


def cpu_baseline(w, budget_s=12.0):
    """The float64 oracle, as it stands, on the host cores: paged attention over the batch."""
    from threadpoolctl import threadpool_limits
    from oracle import attention as oa
    from oracle import run as orun

    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    t0 = time.perf_counter()
    rp = orun.replay(w)
    log(f"[bench] oracle replay built in {time.perf_counter() - t0:.1f}s")
    s = w.spec
    order = np.random.default_rng(0).permutation(w.num_seqs)
    done, tokens, elapsed, passes = 0, 0, 0.0, 0
    with threadpool_limits(limits=cores):
        while elapsed < budget_s:
            for i in order:
                t = time.perf_counter()
                oa.paged_attention(w.q, rp.k_cache, rp.v_cache, rp.tables, rp.context_lens, w.scale, s.kv_dtype,
                                   seqs=[int(i)])
                elapsed += time.perf_counter() - t
                done += 1
                tokens += int(w.context_lens[i])
                if elapsed >= budget_s:
                    break
            passes += 1
    kv = tokens * w.kv_bytes_per_token
    return {"value": kv / elapsed / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "seq_steps_per_s": done / elapsed,
            "sample": f"{done} sequence-steps over {passes} pass(es) of the {w.num_seqs}-sequence {s.name} batch "
                      f"({tokens} context tokens), float64 NumPy "
                      f"oracle (gather through the block table, then softmax(qK^T*scale)V), BLAS threads={cores}, "
                      f"{elapsed:.1f}s"}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
HOST_LINK_PEAK_GBPS = 63.0  # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes, 128b/130b coding


def measure_swap(stream, block_tokens=(1, 4, 16, 32), per_cache=256 << 20):
    """Preemption by swapping, at the Llama-7B layer shape (H_kv 32, d 128, bf16): move per_cache bytes of
    scattered device blocks of each cache to consecutive page-locked host blocks and back, with pkv_swap_blocks
    (one launch for every block of both caches) and with one DMA copy per block (hipMemcpyAsync through torch,
    whose per-call host cost is part of what it measures), at several block sizes; one contiguous DMA copy of
    the same bytes gives the link's ceiling."""
    import torch
    from paged_kv_cache_physical_amd import pkv_swap_blocks
    H, d = 32, 128
    rng = np.random.default_rng(0)
    out = {}
    for bt in block_tokens:
        bb = bt * H * d * 2  # bytes of one block of one cache
        n = per_cache // bb
        dk = torch.zeros((2 * n, bb // 2), dtype=torch.bfloat16, device="cuda")
        dv = torch.zeros_like(dk)
        hk = torch.zeros((n, bb // 2), dtype=torch.bfloat16).pin_memory()
        hv = torch.zeros((n, bb // 2), dtype=torch.bfloat16).pin_memory()
        src = rng.choice(2 * n, size=n, replace=False)
        p_out = np.stack([src, np.arange(n)], 1).astype(np.int32)
        p_in = np.ascontiguousarray(p_out[:, ::-1])
        po, pi = torch.from_numpy(p_out).cuda(), torch.from_numpy(p_in).cuda()
        moved = 2 * n * bb
        with torch.cuda.stream(stream):
            k_out = time_launches(lambda: pkv_swap_blocks(dk, dv, hk, hv, po, stream), 4, stream)
            k_in = time_launches(lambda: pkv_swap_blocks(hk, hv, dk, dv, pi, stream), 4, stream)

            def dma(pairs, sk, sv, tk, tv):
                for i, j in pairs.tolist():
                    tk[j].copy_(sk[i], non_blocking=True)
                    tv[j].copy_(sv[i], non_blocking=True)

            d_out = time_launches(lambda: dma(p_out, dk, dv, hk, hv), 1, stream)
            d_in = time_launches(lambda: dma(p_in, hk, hv, dk, dv), 1, stream)

            def bulk(sk, sv, tk, tv):  # one contiguous copy per cache: the DMA engines' own ceiling
                tk[:n].copy_(sk[:n], non_blocking=True)
                tv[:n].copy_(sv[:n], non_blocking=True)

            b_out = time_launches(lambda: bulk(dk, dv, hk, hv), 4, stream)
            b_in = time_launches(lambda: bulk(hk, hv, dk, dv), 4, stream)
        torch.cuda.synchronize()
        gbps = lambda ms: moved / (ms * 1e-3) / 1e9
        out[f"block_tokens_{bt}"] = {
            "block_bytes": bb, "blocks_per_cache": n, "bytes_each_way": moved,
            "kernel_out_gbps": round(gbps(k_out[1]), 2), "kernel_in_gbps": round(gbps(k_in[1]), 2),
            "dma_per_block_out_gbps": round(gbps(d_out[0]), 2), "dma_per_block_in_gbps": round(gbps(d_in[0]), 2),
            "dma_contiguous_out_gbps": round(gbps(b_out[1]), 2), "dma_contiguous_in_gbps": round(gbps(b_in[1]), 2),
            "kernel_out_us": round(1e3 * k_out[1], 1), "kernel_in_us": round(1e3 * k_in[1], 1)}
        log(f"[bench] swap, {bt}-token blocks: {json.dumps(out[f'block_tokens_{bt}'])}")
        del dk, dv, hk, hv, po, pi
        torch.cuda.empty_cache()
    return {"shape": "H_kv 32, d 128, bf16, both caches", "host_link_peak_gbps": HOST_LINK_PEAK_GBPS, **out}


# Runs of causal queries (pkv_paged_attention_multi).  Each case: name -> (sequences, H_q, H_kv, context lengths
# (lo, hi) uniform, or a constant, run length per sequence (an int, or "all" for the whole prompt)).
MULTI_CASES = {
    "verify4_llama7b_bf16": (64, 32, 32, (128, 2048), 4),
    "verify4_gqa_bf16": (256, 64, 8, (128, 2048), 4),
    "verify4_long_bf16": (8, 32, 8, 32768, 4),
    "prefill2048_gqa_bf16": (16, 32, 8, 2048, "all"),
    "prefix_tail256_gqa_bf16": (64, 32, 8, 1280, 256),
    # one continuous-batching step: 4 sequences take a 512-token prompt chunk, 60 decode one token
    "mixed4x512_plus60_gqa_bf16": (64, 32, 8, (640, 2048), ("mixed", 4, 512)),
}
# --multi-sweep: the verification batches with 1, 2, 4 or 8 drafted tokens per sequence (how the cost of a run
# grows with its length, against the decode kernel on the same kind of batch).
SWEEP_CASES = {f"verify{k}_llama7b_bf16": (64, 32, 32, (128, 2048), k) for k in (1, 2, 4, 8)}
SWEEP_CASES.update({f"verify{k}_gqa_bf16": (256, 64, 8, (128, 2048), k) for k in (1, 4)})


def measure_multi(stream, reps=20, case=None, cases=None):
    """pkv_paged_attention_multi on synthetic batches (bf16 caches, d 128, B 16, shuffled pool, every valid slot
    N(0, 1)).  Verification runs are reported as KV GB/s (each sequence's K/V bytes counted once) against HBM
    peak; prompt runs as matrix-core TFLOP/s (4 d flop per visible (query head, token) pair: QK and PV) against
    the dense bf16 peak."""
    import torch
    import paged_kv_cache_physical_amd as pk
    d, B = 128, 16
    out = {}
    for name, (S, Hq, Hkv, lens_spec, run) in (MULTI_CASES if cases is None else cases).items():
        if case is not None and name != case:
            continue
        rng = np.random.default_rng(1)
        lens = (rng.integers(lens_spec[0], lens_spec[1], size=S, endpoint=True) if isinstance(lens_spec, tuple)
                else np.full(S, lens_spec)).astype(np.int64)
        if run == "all":
            runs = lens.copy()
        elif isinstance(run, tuple):  # ("mixed", k, chunk): k sequences run `chunk` queries, the rest one
            runs = np.ones(S, dtype=np.int64)
            runs[:run[1]] = run[2]
        else:
            runs = np.full(S, run, dtype=np.int64)
        nb = int(sum(-(-int(n) // B) for n in lens))
        pool = pk.Pool(nb, B, rng.permutation(nb).astype(np.int32))
        ids = [pool.create() for _ in range(S)]
        pool.append(ids, lens.tolist())
        tables, clens = pool.block_tables(ids, int(max(-(-int(n) // B) for n in lens)))
        kc, vc = pk.empty_caches(nb, Hkv, B, d, "bf16", poison=False)
        kc.normal_()
        vc.normal_()
        T = int(runs.sum())
        q = torch.randn((T, Hq, d), device="cuda").to(torch.bfloat16)
        o = torch.empty((T, Hq, d), dtype=torch.float32, device="cuda")
        starts = torch.from_numpy(np.concatenate([[0], np.cumsum(runs)]).astype(np.int32)).cuda()
        bt, cl = torch.from_numpy(tables).cuda(), torch.from_numpy(clens).cuda()
        wsb = pk.pkv_attention_multi_workspace_bytes(S, Hq, Hkv, d, int(lens.max()), int(runs.max()))
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
        # longest first: the order a scheduler that knows the lengths hands over
        order = torch.from_numpy(np.argsort(-lens, kind="stable").astype(np.int32)).cuda()
        fn = lambda: pk.pkv_paged_attention_multi(o, q, kc, vc, bt, cl, starts, int(lens.max()), int(runs.max()),
                                                  1.0 / np.sqrt(d), stream, workspace=ws, seq_order=order)
        with torch.cuda.stream(stream):
            for _ in range(3):
                fn()
            t = time_launches(fn, reps, stream)
        us = 1e3 * t[0]
        visible = int(sum(int(r) * int(n) - int(r) * (int(r) - 1) // 2 for n, r in zip(lens, runs)))
        flops = 4 * d * Hq * visible
        kv_bytes = int(lens.sum()) * 2 * Hkv * d * 2
        rec = {"sequences": S, "H_q": Hq, "H_kv": Hkv, "context_tokens": int(lens.sum()), "query_rows": T,
               "workspace_bytes": wsb,
               "launch_us": round(us, 2), "launch_us_median": round(1e3 * t[1], 2),
               "kv_bytes": kv_bytes, "kv_gbps": round(kv_bytes / (us * 1e-6) / 1e9, 1),
               "flops": flops, "tflops": round(flops / (us * 1e-6) / 1e12, 2)}
        if isinstance(run, tuple):  # mixed work: both fractions, neither bound alone
            rec["hbm_frac"] = round(rec["kv_gbps"] / HBM_PEAK_GBPS, 4)
            rec["mfma_frac"] = round(rec["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
            rec["roofline"] = {"bound": "mixed", "achieved": rec["kv_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                               "frac": rec["hbm_frac"]}
        elif run == "all" or run > 16:
            rec["roofline"] = {"bound": "mfma", "achieved": rec["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(rec["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)}
        else:
            rec["roofline"] = {"bound": "hbm", "achieved": rec["kv_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                               "frac": round(rec["kv_gbps"] / HBM_PEAK_GBPS, 4)}
        out[name] = rec
        log(f"[bench] multi {name}: {json.dumps(rec)}")
        del kc, vc, q, o, ws, order
        torch.cuda.empty_cache()
    return out


def copy_probe(stream, nbytes=1 << 30):
    """A plain device copy of known size (reads and writes nbytes): the reference dispatch that
    scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    with torch.cuda.stream(stream):
        for _ in range(3):
            y.copy_(x)
    torch.cuda.synchronize()
    del x, y
    torch.cuda.empty_cache()


def decode_kernel_flags(kernel_name: str):
    """(LIST, WRITE, FUSED) template flags of a paged_decode_kernel name (arguments DT, D, G, B, LIST, WRITE,
    FUSED, queries per item), or None for another kernel."""
    if "paged_decode_kernel<" not in kernel_name:
        return None
    args = [x.strip() for x in kernel_name.split("paged_decode_kernel<", 1)[1].split(">", 1)[0].split(",")]
    return tuple(x == "true" for x in args[4:7])


def is_step_kernel(kernel_name: str) -> bool:
    """The decode step's kernel: item list, token write and in-kernel combination."""
    return decode_kernel_flags(kernel_name) == (True, True, True)


def traffic_summary(pmc_dirs, workload: str, nbytes=1 << 30):
    """HBM bytes per decode-step kernel dispatch from rocprofv3 --pmc CSVs (one run with FETCH_SIZE, one with
    WRITE_SIZE), each counter scaled by its reading on the copy probe of nbytes."""
    import csv
    import glob
    vals = {}
    for d in pmc_dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                name, ctr = r["Kernel_Name"], r["Counter_Name"]
                kind = ("decode" if is_step_kernel(name) else
                        "copy" if "copy" in name.lower() else None)
                if kind is None:
                    continue
                gsize = int(r.get("Grid_Size", 0) or 0)
                vals.setdefault((kind, ctr), []).append((gsize, float(r["Counter_Value"])))
    out = {"workload": workload, "kernel_source_sha": kernel_sha()}
    for ctr, key in (("FETCH_SIZE", "read"), ("WRITE_SIZE", "write")):
        dec = [v for _, v in vals.get(("decode", ctr), [])]
        cpy = [v for _, v in vals.get(("copy", ctr), [])]
        if not dec or not cpy:
            continue
        cpy_kib = float(np.median(sorted(cpy)[-3:]))  # the three copies of nbytes (largest readings)
        scale = nbytes / (cpy_kib * 1024.0)
        out[f"{key}_scale"] = scale
        out[f"{key}_bytes_per_launch"] = float(np.median(dec)) * 1024.0 * scale
        out[f"{key}_dispatches"] = len(dec)
    if "read_bytes_per_launch" in out:
        out["hbm_bytes_per_launch"] = out["read_bytes_per_launch"] + out.get("write_bytes_per_launch", 0.0)
    return out


def kernel_counters(pmc_dirs, nbytes=1 << 30):
    """Per-kernel medians of every counter in rocprofv3 --pmc CSVs (rows: kernel and grid size, dispatches,
    counters).
    FETCH_SIZE / WRITE_SIZE also as bytes per dispatch, scaled by their readings on the copy probe when the
    inputs hold it (the probe's three 1 GiB copies)."""
    import csv
    import glob
    vals = {}
    for d in pmc_dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                key = (r["Kernel_Name"], int(r.get("Grid_Size", 0) or 0))  # one row per kernel and launch size
                vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    scale = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        # the probe: of the copy kernels' three largest readings, the largest median (the runtime's copy of nbytes)
        top = [float(np.median(sorted(c[ctr])[-3:])) for (name, _), c in vals.items()
               if "copy" in name.lower() and ctr in c and len(c[ctr]) >= 3]
        if top:
            scale[ctr] = nbytes / (max(top) * 1024.0)
    rows = []
    for (name, grid), ctrs in sorted(vals.items()):
        rec = {"kernel": name, "grid_size": grid, "dispatches": max(len(v) for v in ctrs.values())}
        for ctr, v in sorted(ctrs.items()):
            rec[ctr] = float(np.median(v))
            if ctr in scale:
                rec[ctr.lower() + "_bytes"] = rec[ctr] * 1024.0 * scale[ctr]
        rows.append(rec)
    return {"scale": scale, "kernels": rows}


def traffic_from_profiles(workload: str):
    path = os.path.join(ROOT, "profiles", f"paged_decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-extra", action="store_true", help="skip the other decode batches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-swap", action="store_true", help="skip the device <-> host swap measurement")
    ap.add_argument("--no-multi", action="store_true", help="skip the runs-of-queries measurement")
    ap.add_argument("--multi-only", action="store_true", help="only the runs-of-queries measurement")
    ap.add_argument("--multi-case", default=None, help="with --multi-only: one case of MULTI_CASES")
    ap.add_argument("--multi-sweep", action="store_true",
                    help="only the verification batches with 1, 2, 4 and 8 drafted tokens (SWEEP_CASES)")
    ap.add_argument("--swap-only", action="store_true",
                    help="run only the swap measurement and print its JSON object (for profiling pkv_swap_blocks)")
    ap.add_argument("--partition", type=int, default=None, help="override the workload's partition size")
    ap.add_argument("--extra", default=",".join(EXTRA), help="comma-separated extra workloads")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (the reference dispatch for rocprofv3 byte counters)")
    ap.add_argument("--kernel-counters", nargs="+", metavar="DIR",
                    help="print per-kernel medians of the counters in rocprofv3 --pmc output dirs (bytes scaled by "
                         "the copy probe when present) and exit")
    ap.add_argument("--traffic-from", nargs="+", metavar="DIR",
                    help="write profiles/paged_decode_<workload>_traffic.json from rocprofv3 --pmc output dirs "
                         "(FETCH_SIZE and WRITE_SIZE runs of this script with --copy-probe) and exit")
    args = ap.parse_args()
    if args.kernel_counters:
        print(json.dumps(kernel_counters(args.kernel_counters), indent=1))
        return
    if args.traffic_from:
        rec = traffic_summary(args.traffic_from, args.workload)
        path = os.path.join(ROOT, "profiles", f"paged_decode_{args.workload}_traffic.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    from paged_kv_cache_physical_amd import _lib

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    _lib.lib()  # fail loudly if the HIP library is not built
    stream = torch.cuda.Stream()  # default priority
    if args.swap_only:
        print(json.dumps(measure_swap(stream)), flush=True)
        return
    if args.multi_sweep:
        print(json.dumps(measure_multi(stream, cases=SWEEP_CASES)), flush=True)
        return
    if args.multi_only:
        print(json.dumps(measure_multi(stream, case=args.multi_case)), flush=True)
        return

    over = {} if args.partition is None else {"partition_size": args.partition}
    w = wl.named(args.workload, seed=0, **over)
    head = measure(w, args.steps, args.warmup, stream)
    log(f"[bench] {w.spec.name}: {json.dumps(head)}")
    extra = {}
    if not args.no_extra:
        for name in [x for x in args.extra.split(",") if x]:
            if name == args.workload:
                continue
            r = measure(wl.named(name, seed=0, **over), 20, 5, stream)
            r["pct_hbm_peak_partition_kernel"] = 100 * r["kv_gbps_partition_kernel"] / HBM_PEAK_GBPS
            extra[name] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}
            log(f"[bench] {name}: {json.dumps(extra[name])}")
    if args.copy_probe:
        copy_probe(stream)
    try:
        head["host_allocator_us_per_step"], head["host_allocator_c_us_per_step"] = host_allocator_step_us(w)
    except Exception as e:  # a full pool cannot take another token per sequence
        log(f"[bench] host allocator step not timed: {e}")
    ceiling = hbm_read_ceiling(stream)
    log(f"[bench] streaming-read probe {ceiling:.0f} GB/s")
    swap = None if args.no_swap else measure_swap(stream)
    multi = None if args.no_multi else measure_multi(stream)
    prefix = measure_prefix_cache()
    log(f"[bench] prefix cache {json.dumps(prefix)}")
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)
    if cpu:
        log(f"[bench] cpu baseline {json.dumps(cpu)}")

    achieved = head["kv_gbps_step_launch"]
    line = {
        "metric": METRIC,
        "value": round(head["kv_gbps_step"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.spec.kv_dtype,
        "data": "synthetic",
        "config": describe(w),
        "seq_steps_per_s": round(head["seq_steps_per_s"], 1),
        "pct_hbm_peak_step": round(100 * head["kv_gbps_step"] / HBM_PEAK_GBPS, 2),
        "host_allocator_us_per_step": round(head.get("host_allocator_us_per_step", float("nan")), 2),
        "host_allocator_c_us_per_step": round(head.get("host_allocator_c_us_per_step", float("nan")), 2),
        "kernels_us": {"decode_step_kernel": round(head["step_us"]["mean"], 2),
                       "two_stage_partition_pass": round(head["partition_kernel_us"]["mean"], 2),
                       "two_stage_reduce": round(head["reduce_kernel_us"], 2),
                       "reshape_and_cache": round(head["reshape_and_cache_us"], 2),
                       "attention_call": round(head["attention_us"], 2),
                       "step_as_separate_calls": round(head["separate_calls_step_us"], 2)},
        "timing_us": {"step_each_launch": {k: round(v, 2) for k, v in head["step_us"].items()},
                      "partition_pass": {k: round(v, 2) for k, v in head["partition_kernel_us"].items()}},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles(w.spec.name),
                     "kernel": "paged_decode_kernel, decode-step variant (token write, attention, in-kernel "
                               "combination: the step's only launch)",
                     "bytes_per_launch": w.kv_bytes,
                     "launch_us": round(head["step_us"]["mean"], 2)},
        "hbm_read_ceiling_gbps": round(ceiling, 1),
        "swap": swap,
        "multi_query": multi,
        "prefix_cache": prefix,
        "cpu_baseline": cpu,
        "other_workloads": extra,
        "kernel_source_sha": kernel_sha(),
        "source_shas": source_shas(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
