"""Seeded synthetic decode workloads for the paged KV-cache decode path.

This module is the only code shared by the product path (the HIP library and
its Python binding) and the oracle.  It draws inputs and nothing else: context
lengths, the shuffled order of the free block pool, query vectors, the key and
value vectors of every token, and the script of allocator operations (create,
fork, append) that builds each batch.  It computes no slot, block table,
softmax or attention value; each side derives those with its own code.

Random streams: every array comes from its own NumPy PCG64 generator seeded by
``SeedSequence(entropy=seed, spawn_key=(stream, *index))``, so any sequence's
tokens can be regenerated alone and in any order.  Values are drawn as float32
N(0, 1); for bf16 caches they are rounded to bfloat16 with round-to-nearest-even
and carried as their 16-bit patterns in ``uint16`` arrays.

The five named workloads follow the decode batches the pages' problem
statement calls for (a tiny fp32 step over the worked example's lengths
37/91/128/201/511, a Llama-7B-shaped MHA batch, a GQA batch with lognormal
lengths, beam search over a shared 1000-token prompt, and long 32768-token
contexts); the sizes of each are in NAMED below.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

# Stream identifiers for SeedSequence spawn keys.
STREAM_LENS = 1
STREAM_PERM = 2
STREAM_Q = 3
STREAM_KV = 4
STREAM_TAIL_LENS = 5
STREAM_TAIL_KV = 6
STREAM_NEW_KV = 7  # the decode step's new token of each sequence
STREAM_STEM = 8  # prefix-sharing requests: stem lengths and token ids
STREAM_STEM_KV = 9  # K/V of a stem's tokens, per (stem, position)
STREAM_REQ = 10  # a request's stem choice, tail length and tail token ids
STREAM_REQ_KV = 11  # K/V of a request's own tail tokens

# Bit patterns used to poison never-written cache slots.  A read that is not
# masked turns the attention output into NaN.
POISON_BF16 = np.uint16(0x7FC0)
POISON_F32 = np.uint32(0x7FC00000)

KV_DTYPES = ("f32", "bf16")


def rng_for(seed: int, *key: int) -> np.random.Generator:
    """Independent PCG64 generator for stream ``key`` of ``seed``."""
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=tuple(int(k) for k in key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are finite normal
    samples, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_values(rng: np.random.Generator, shape, kv_dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if kv_dtype == "f32":
        return x
    if kv_dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def value_itemsize(kv_dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[kv_dtype]


def storage_dtype(kv_dtype: str):
    return {"f32": np.float32, "bf16": np.uint16}[kv_dtype]


# ---------------------------------------------------------------------------
# Allocator scripts
# ---------------------------------------------------------------------------


@dataclass
class Create:
    """Create ``count`` empty sequences; ids are assigned 0, 1, 2, ... in creation order."""

    count: int


@dataclass
class Fork:
    """Create one child sequence that shares every block of ``parent``."""

    parent: int


@dataclass
class Append:
    """Append ``counts[i]`` tokens to ``seqs[i]`` (all or nothing).

    ``values()`` returns ``(k, v)`` of shape ``[sum(counts)][H_kv][d]`` in
    sequence-major order: all new tokens of ``seqs[0]`` first, in position
    order, then those of ``seqs[1]``, and so on.
    """

    seqs: np.ndarray
    counts: np.ndarray
    values: Callable[[], Tuple[np.ndarray, np.ndarray]] = field(repr=False)
    decode: bool = False  # True for the final one-token-per-sequence decode step


@dataclass(frozen=True)
class Spec:
    name: str
    kind: str  # "decode" or "beam"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str
    partition_size: int
    seed: int = 0
    # decode kind
    lens: Optional[Tuple[int, ...]] = None  # fixed lengths, else drawn by ``len_dist``
    len_dist: Optional[Tuple] = None  # ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi) | ("const", n)
    num_blocks: Optional[int] = None  # pool size; None -> ceil(pool_factor * blocks used)
    pool_factor: float = 1.1
    # beam kind
    prompts: int = 0
    beams: int = 0
    prefix_len: int = 0
    tail_range: Tuple[int, int] = (1, 1)


class Workload:
    """One seeded decode batch: shapes, pool order, q, per-token K/V and the allocator script."""

    def __init__(self, spec: Spec):
        if spec.kv_dtype not in KV_DTYPES:
            raise ValueError(spec.kv_dtype)
        if spec.num_q_heads % spec.num_kv_heads:
            raise ValueError("num_q_heads must be a multiple of num_kv_heads")
        self.spec = spec
        s = spec
        if s.kind == "decode":
            self.context_lens = self._draw_lens()
            self.num_seqs = s.num_seqs
        elif s.kind == "beam":
            tails = rng_for(s.seed, STREAM_TAIL_LENS).integers(
                s.tail_range[0], s.tail_range[1], size=(s.prompts, s.beams), endpoint=True)
            self.tail_lens = tails.astype(np.int32)
            self.context_lens = (s.prefix_len + self.tail_lens).reshape(-1).astype(np.int32)
            self.num_seqs = s.prompts * s.beams
        else:
            raise ValueError(s.kind)
        B = s.block_size
        used = int(np.sum((self.context_lens.astype(np.int64) + B - 1) // B))
        self.blocks_needed_private = used
        if s.num_blocks is not None:
            self.num_blocks = int(s.num_blocks)
        else:
            self.num_blocks = int(math.ceil(s.pool_factor * used))
        self.free_order = rng_for(s.seed, STREAM_PERM).permutation(self.num_blocks).astype(np.int32)
        self.scale = np.float32(1.0 / math.sqrt(s.head_dim))
        self.q = draw_values(rng_for(s.seed, STREAM_Q), (self.num_seqs, s.num_q_heads, s.head_dim), s.kv_dtype)
        self.max_context_len = int(self.context_lens.max()) if self.num_seqs else 0
        self.total_tokens = int(self.context_lens.astype(np.int64).sum())

    # -- lengths ---------------------------------------------------------
    def _draw_lens(self) -> np.ndarray:
        s = self.spec
        if s.lens is not None:
            lens = np.asarray(s.lens, dtype=np.int64)
            if len(lens) != s.num_seqs:
                raise ValueError("lens length != num_seqs")
            return lens.astype(np.int32)
        rng = rng_for(s.seed, STREAM_LENS)
        d = s.len_dist
        if d[0] == "uniform":
            lens = rng.integers(d[1], d[2], size=s.num_seqs, endpoint=True)
        elif d[0] == "lognormal":
            median, sigma, lo, hi = d[1:]
            lens = np.clip(np.rint(rng.lognormal(mean=math.log(median), sigma=sigma, size=s.num_seqs)), lo, hi)
        elif d[0] == "const":
            lens = np.full(s.num_seqs, d[1])
        else:
            raise ValueError(d)
        return lens.astype(np.int32)

    # -- values ------------------------------------------------------------
    def _token_block(self, key: Tuple[int, ...], n: int) -> Tuple[np.ndarray, np.ndarray]:
        s = self.spec
        rng = rng_for(s.seed, *key)
        shape = (n, s.num_kv_heads, s.head_dim)
        k = draw_values(rng, shape, s.kv_dtype)
        v = draw_values(rng, shape, s.kv_dtype)
        return k, v

    def token_kv(self, seq: int) -> Tuple[np.ndarray, np.ndarray]:
        """Logical (contiguous, position-ordered) K and V of sequence ``seq``: ``[n][H_kv][d]``.

        Positions before the last come from the sequence's context stream (the
        shared prompt stream plus the beam's own tail stream for beam search);
        the last position is the decode step's new token, drawn from its own
        stream.
        """
        s = self.spec
        kn, vn = self._token_block((STREAM_NEW_KV, seq), 1)
        if s.kind == "decode":
            kc, vc = self._token_block((STREAM_KV, seq), int(self.context_lens[seq]) - 1)
            return np.concatenate([kc, kn]), np.concatenate([vc, vn])
        p, b = divmod(seq, s.beams)
        kp, vp = self._token_block((STREAM_KV, p), s.prefix_len)
        kt, vt = self._token_block((STREAM_TAIL_KV, p, b), int(self.tail_lens[p, b]) - 1)
        return np.concatenate([kp, kt, kn]), np.concatenate([vp, vt, vn])

    def _gather_tokens(self, pieces: Sequence[Tuple[Tuple[int, ...], int, int, int]]) -> Tuple[np.ndarray, np.ndarray]:
        """Concatenate token ranges ``(key, n_total, lo, hi)`` of several streams, drawn in parallel."""
        s = self.spec
        total = sum(hi - lo for _, _, lo, hi in pieces)
        dt = storage_dtype(s.kv_dtype)
        k_out = np.empty((total, s.num_kv_heads, s.head_dim), dtype=dt)
        v_out = np.empty_like(k_out)
        offs = np.cumsum([0] + [hi - lo for _, _, lo, hi in pieces])

        def work(i):
            key, n, lo, hi = pieces[i]
            if hi <= lo:
                return
            k, v = self._token_block(key, n)
            k_out[offs[i]:offs[i + 1]] = k[lo:hi]
            v_out[offs[i]:offs[i + 1]] = v[lo:hi]

        threads = min(16, os.cpu_count() or 1, max(1, len(pieces)))
        if threads > 1 and total * s.num_kv_heads * s.head_dim > 1_000_000:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(work, range(len(pieces))))
        else:
            for i in range(len(pieces)):
                work(i)
        return k_out, v_out

    # -- allocator script ---------------------------------------------------
    def script(self) -> List[object]:
        """Allocator operations that build the batch; the last op is the decode step."""
        s = self.spec
        S = self.num_seqs
        ops: List[object] = []
        if s.kind == "decode":
            lens = self.context_lens.astype(np.int64)
            seqs = np.arange(S, dtype=np.int32)
            ops.append(Create(S))
            pre = [((STREAM_KV, i), int(lens[i]) - 1, 0, int(lens[i]) - 1) for i in range(S)]
            dec = [((STREAM_NEW_KV, i), 1, 0, 1) for i in range(S)]
            ops.append(Append(seqs, (lens - 1).astype(np.int32), lambda pre=pre: self._gather_tokens(pre)))
            ops.append(Append(seqs, np.ones(S, np.int32), lambda dec=dec: self._gather_tokens(dec), decode=True))
            return ops
        # beam search: each prompt is prefilled once and forked beams-1 times;
        # beam b of prompt p is sequence p*beams + b (beam 0 is the parent).
        for p in range(s.prompts):
            ops.append(Create(1))
            pid = p * s.beams
            piece = [((STREAM_KV, p), s.prefix_len, 0, s.prefix_len)]
            ops.append(Append(np.array([pid], np.int32), np.array([s.prefix_len], np.int32),
                              lambda piece=piece: self._gather_tokens(piece)))
            for _ in range(s.beams - 1):
                ops.append(Fork(pid))
        seqs = np.arange(S, dtype=np.int32)
        tails = self.tail_lens.reshape(-1).astype(np.int64)
        pre, dec = [], []
        for i in range(S):
            p, b = divmod(i, s.beams)
            pre.append(((STREAM_TAIL_KV, p, b), int(tails[i]) - 1, 0, int(tails[i]) - 1))
            dec.append(((STREAM_NEW_KV, i), 1, 0, 1))
        ops.append(Append(seqs, (tails - 1).astype(np.int32), lambda pre=pre: self._gather_tokens(pre)))
        ops.append(Append(seqs, np.ones(S, np.int32), lambda dec=dec: self._gather_tokens(dec), decode=True))
        return ops

    # -- sizes ---------------------------------------------------------------
    @property
    def kv_bytes_per_token(self) -> int:
        s = self.spec
        return 2 * s.num_kv_heads * s.head_dim * value_itemsize(s.kv_dtype)

    @property
    def kv_bytes(self) -> int:
        """Bytes of valid K and V tokens one decode step reads (padding excluded)."""
        return self.total_tokens * self.kv_bytes_per_token

    def block_shape(self) -> Tuple[int, int, int]:
        s = self.spec
        return (s.num_kv_heads, s.block_size, s.head_dim)


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------

NAMED = {
    "tiny_f32": Spec("tiny_f32", "decode", num_seqs=5, num_q_heads=8, num_kv_heads=8, head_dim=64,
                     block_size=16, kv_dtype="f32", partition_size=0, lens=(37, 91, 128, 201, 511),
                     num_blocks=128),
    "llama7b_bf16": Spec("llama7b_bf16", "decode", num_seqs=64, num_q_heads=32, num_kv_heads=32, head_dim=128,
                         block_size=16, kv_dtype="bf16", partition_size=512, len_dist=("uniform", 128, 2048),
                         num_blocks=16384),
    "gqa_bf16_b16": Spec("gqa_bf16_b16", "decode", num_seqs=256, num_q_heads=64, num_kv_heads=8, head_dim=128,
                         block_size=16, kv_dtype="bf16", partition_size=512,
                         len_dist=("lognormal", 1024, 0.8, 16, 8192), pool_factor=1.1),
    "gqa_bf16_b32": Spec("gqa_bf16_b32", "decode", num_seqs=256, num_q_heads=64, num_kv_heads=8, head_dim=128,
                         block_size=32, kv_dtype="bf16", partition_size=512,
                         len_dist=("lognormal", 1024, 0.8, 16, 8192), pool_factor=1.1),
    "beam_cow_bf16": Spec("beam_cow_bf16", "beam", num_seqs=128, num_q_heads=32, num_kv_heads=8, head_dim=128,
                          block_size=16, kv_dtype="bf16", partition_size=512, num_blocks=16384,
                          prompts=32, beams=4, prefix_len=1000, tail_range=(1, 256)),
    "long_bf16": Spec("long_bf16", "decode", num_seqs=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=16, kv_dtype="bf16", partition_size=512, len_dist=("const", 32768),
                      num_blocks=16384),
}


def named(name: str, seed: int = 0, **overrides) -> Workload:
    spec = replace(NAMED[name], seed=seed, **overrides)
    return Workload(spec)


def small_decode(num_seqs: int, lens_range: Tuple[int, int], num_q_heads: int, num_kv_heads: int,
                 head_dim: int, block_size: int, kv_dtype: str, partition_size: int = 0,
                 seed: int = 0, pool_factor: float = 1.5, lens: Optional[Sequence[int]] = None,
                 num_blocks: Optional[int] = None) -> Workload:
    """A small ragged decode batch for parity tests."""
    spec = Spec("small", "decode", num_seqs=num_seqs, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                head_dim=head_dim, block_size=block_size, kv_dtype=kv_dtype, partition_size=partition_size,
                seed=seed, lens=tuple(lens) if lens is not None else None,
                len_dist=None if lens is not None else ("uniform", lens_range[0], lens_range[1]),
                pool_factor=pool_factor, num_blocks=num_blocks)
    return Workload(spec)


@dataclass
class PrefixRequests:
    """Requests whose prompts start with one of a few shared stems (a system prompt, a few-shot header).

    Request r's prompt is ``stems[stem_of[r]]`` followed by its own tail.  A
    token's key and value depend on the run of tokens up to it, so every stem
    token carries the same K/V in every request that shares the stem (drawn
    per (stem, position)), and tail tokens carry the request's own.  Token ids
    are small integers; K/V are N(0, 1) in the cache dtype.  Inputs only:
    which blocks are shared is for each side's allocator to find.
    """

    seed: int
    num_requests: int
    num_stems: int
    stem_range: Tuple[int, int]
    tail_range: Tuple[int, int]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str
    vocab: int = 32000

    def __post_init__(self):
        rs = rng_for(self.seed, STREAM_STEM)
        lo, hi = self.stem_range
        self.stems = [[int(t) for t in rs.integers(0, self.vocab, size=int(rs.integers(lo, hi + 1)))]
                      for _ in range(self.num_stems)]
        self.stem_of, self.tails = [], []
        for r in range(self.num_requests):
            rr = rng_for(self.seed, STREAM_REQ, r)
            self.stem_of.append(int(rr.integers(0, self.num_stems)))
            n = int(rr.integers(self.tail_range[0], self.tail_range[1] + 1))
            self.tails.append([int(t) for t in rr.integers(0, self.vocab, size=n)])

    def prompt(self, r: int) -> List[int]:
        return self.stems[self.stem_of[r]] + self.tails[r]

    def kv(self, r: int) -> Tuple[np.ndarray, np.ndarray]:
        """K and V ``[n][H_kv][d]`` (storage dtype) of every prompt token of request r."""
        shape = (self.num_kv_heads, self.head_dim)
        st = self.stem_of[r]
        k = [draw_values(rng_for(self.seed, STREAM_STEM_KV, st, 0), (len(self.stems[st]),) + shape, self.kv_dtype),
             draw_values(rng_for(self.seed, STREAM_REQ_KV, r, 0), (len(self.tails[r]),) + shape, self.kv_dtype)]
        v = [draw_values(rng_for(self.seed, STREAM_STEM_KV, st, 1), (len(self.stems[st]),) + shape, self.kv_dtype),
             draw_values(rng_for(self.seed, STREAM_REQ_KV, r, 1), (len(self.tails[r]),) + shape, self.kv_dtype)]
        return np.concatenate(k), np.concatenate(v)

    def q(self) -> np.ndarray:
        """One query per request ``[R][H_q][d]`` (storage dtype)."""
        return draw_values(rng_for(self.seed, STREAM_Q), (self.num_requests, self.num_q_heads, self.head_dim),
                           self.kv_dtype)
