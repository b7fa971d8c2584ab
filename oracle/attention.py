"""Decode attention in float64 (test infrastructure; see oracle/__init__).

The pages never print the attention formula; they state that attention needs
the key and value of every earlier token ([P4] KV-cache introduction), that
paging changes how the cache is stored and addressed but not what attention
reads ([P3] section 1), that the kernel reads a sequence's scattered blocks
through its block table ([P2] key technical point 1), and that correctness is
checked against the output of a contiguous-KV baseline ([P3] "Verification
protocol").  GQA/MQA change only the number of KV heads ([P3] section 1).

So the oracle is the plain definition, one sequence at a time:
    g = h // G   (G = H_q / H_kv, contiguous head groups)
    s_t = scale * <q_h, K[t, g]>      for t < n
    out_h = sum_t softmax(s)_t * V[t, g]
computed in float64 from the exact stored bits, softmax taken in two passes
with the maximum subtracted.  ``scale`` is the float32 value the library
receives, widened to float64.

``paged_attention_multi`` is the same definition for several queries per
sequence, each at its own position: the last q_s positions of a sequence of n_s
tokens (all of them already written to the cache) form a run of queries, and
the query at position p sees tokens t <= p only.  A run of q_s = n_s is the
prompt's own attention (the prefill that computes a whole prompt's KV in one
pass, [P4] "Preemption", recomputation); a short run over a longer context is
what speculative decoding verifies before it keeps or rolls back the staged
positions, and what a prompt whose leading blocks came from the prefix cache
computes for its remaining tokens ([P3] section 5: blockwise attention and
paging compose; speculative decoding stages and rolls back KV positions).

``attention_split`` is the split-context form: each partition of P tokens
yields (m_p, l_p, acc_p) = (max s, sum e^(s - m_p), sum e^(s - m_p) v) and the
results combine as out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p with
M = max_p m_p.  Blockwise softmax of this kind is the organisation the
FlashAttention reference in [P3] section 5 points to; it equals the direct
softmax exactly in real arithmetic.
"""

from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from . import cache as _cache


def attention_contiguous(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """out[H_q][d] for one sequence; q ``[H_q][d]``, k and v ``[n][H_kv][d]`` (float64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, d = q.shape
    n, Hkv, _ = k.shape
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    if n == 0:
        raise ValueError("empty context")
    G = Hq // Hkv
    out = np.empty((Hq, d), dtype=np.float64)
    sc = float(np.float64(scale))
    for h in range(Hq):
        g = h // G
        s = sc * (k[:, g, :] @ q[h])
        w = np.exp(s - s.max())
        out[h] = (w @ v[:, g, :]) / w.sum()
    return out


def partials(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, partition_size: int
             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per-partition (m [P][H_q], l [P][H_q], acc [P][H_q][d]) for one sequence (natural exp)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, d = q.shape
    n, Hkv, _ = k.shape
    G = Hq // Hkv
    npart = -(-n // partition_size)
    m = np.empty((npart, Hq))
    l = np.empty((npart, Hq))
    acc = np.empty((npart, Hq, d))
    sc = float(np.float64(scale))
    for p in range(npart):
        lo, hi = p * partition_size, min(n, (p + 1) * partition_size)
        for h in range(Hq):
            g = h // G
            s = sc * (k[lo:hi, g, :] @ q[h])
            m[p, h] = s.max()
            w = np.exp(s - m[p, h])
            l[p, h] = w.sum()
            acc[p, h] = w @ v[lo:hi, g, :]
    return m, l, acc


def combine(m: np.ndarray, l: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """Log-sum-exp combination of per-partition results into out[H_q][d]."""
    M = m.max(axis=0)
    w = np.exp(m - M)  # [P][H_q]
    return (w[:, :, None] * acc).sum(axis=0) / (w * l).sum(axis=0)[:, None]


def attention_split(q, k, v, scale: float, partition_size: int) -> np.ndarray:
    m, l, acc = partials(q, k, v, scale, partition_size)
    return combine(m, l, acc)


def paged_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
                    context_lens: Sequence[int], scale: float, kv_dtype: str,
                    seqs: Sequence[int] = None) -> np.ndarray:
    """out[S][H_q][d] (float64): gather each sequence through its table, then contiguous attention.

    ``q`` is ``[S][H_q][d]`` in the cache's storage dtype; only ``seqs`` (all by
    default) are computed, the other rows are NaN.
    """
    S, Hq, d = q.shape
    out = np.full((S, Hq, d), np.nan)
    rows = range(S) if seqs is None else seqs
    for s in rows:
        n = int(context_lens[s])
        k, v = _cache.gather(k_cache, v_cache, block_tables[s], n)
        out[s] = attention_contiguous(_cache.to_f64(q[s], kv_dtype), _cache.to_f64(k, kv_dtype),
                                      _cache.to_f64(v, kv_dtype), scale)
    return out


def paged_attention_multi(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
                          context_lens: Sequence[int], query_start: Sequence[int], scale: float,
                          kv_dtype: str) -> np.ndarray:
    """out[T][H_q][d] (float64) for runs of queries over paged K/V.

    Sequence s owns query rows ``query_start[s] .. query_start[s+1] - 1``
    (``q`` is ``[T][H_q][d]`` in the cache's storage dtype); they are its last
    q_s positions n_s - q_s .. n_s - 1, and row i of the run (position
    p = n_s - q_s + i) attends to tokens 0 .. p of the sequence, read through
    its block table.  Written out as that definition in matrix form: gather,
    then per query head the scores of every query of the run against every
    token (one matrix product), -inf where t > p, a softmax along each row with
    its maximum subtracted, and the weighted sum of the values.
    """
    T, Hq, d = q.shape
    out = np.full((T, Hq, d), np.nan)
    starts = [int(x) for x in query_start]
    sc = float(np.float64(scale))
    for s in range(len(starts) - 1):
        n = int(context_lens[s])
        qs = starts[s + 1] - starts[s]
        if qs < 0 or qs > n:
            raise ValueError("a run of queries longer than its context")
        if qs == 0:
            continue
        k, v = _cache.gather(k_cache, v_cache, block_tables[s], n)
        k = _cache.to_f64(k, kv_dtype)
        v = _cache.to_f64(v, kv_dtype)
        Hkv = k.shape[1]
        if Hq % Hkv:
            raise ValueError("H_q must be a multiple of H_kv")
        G = Hq // Hkv
        rows = slice(starts[s], starts[s + 1])
        qq = _cache.to_f64(q[rows], kv_dtype)  # [q_s][H_q][d]
        pos = np.arange(n - qs, n)  # the run's positions
        visible = np.arange(n)[None, :] <= pos[:, None]  # [q_s][n]: token t is seen at position p iff t <= p
        for h in range(Hq):
            g = h // G
            sco = np.where(visible, sc * (qq[:, h, :] @ k[:, g, :].T), -np.inf)
            w = np.exp(sco - sco.max(axis=1, keepdims=True))
            out[rows, h] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out
