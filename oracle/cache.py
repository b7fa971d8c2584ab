"""Physical KV-cache layout, scatter, block copy and gather (test infrastructure; see oracle/__init__).

The pages fix the logical structure: the cache is cut into fixed blocks of B
tokens, a block table maps logical block i to a physical block, and the kernel
reads a sequence's scattered blocks through that table ([P2] core idea items
1-3 and key technical point 1; [P4] KV block figure).  They leave the byte
layout open.  The layout used by the library's interface (and restated here
from that interface's definition, not from its code) is, per cache:

  key cache    K[num_blocks][H_kv][d / X][B][X],  X = 16 / bytes_per_scalar
  value cache  V[num_blocks][H_kv][d][B]

i.e. each (block, KV head) owns one contiguous tile; in the key tile a token's
d values are stored as d / X pieces of 16 bytes, piece j of every token of the
block lying together; the value tile is transposed, one row of B token values
per head dimension.  Token position t of a sequence with table ``bt`` is in
block ``bt[t // B]`` at offset ``t % B``; slot = block * B + offset.

Arrays are NumPy arrays of the storage dtype (float32, or uint16 holding
bfloat16 bits), so copies and scatters move exact bit patterns.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

POISON = {"f32": np.uint32(0x7FC00000), "bf16": np.uint16(0x7FC0)}
_STORE = {"f32": np.float32, "bf16": np.uint16}
_ITEM = {"f32": 4, "bf16": 2}


def key_piece(kv_dtype: str) -> int:
    """X: scalars per 16-byte piece of a key row."""
    return 16 // _ITEM[kv_dtype]


def empty_caches(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, kv_dtype: str
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Key and value caches with every slot set to the NaN poison pattern."""
    X = key_piece(kv_dtype)
    if head_dim % X:
        raise ValueError("head_dim * bytes_per_scalar must be a multiple of 16")
    k = np.empty((num_blocks, num_kv_heads, head_dim // X, block_size, X), dtype=_STORE[kv_dtype])
    v = np.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=_STORE[kv_dtype])
    pattern = POISON[kv_dtype]
    k.view(pattern.dtype)[...] = pattern
    v.view(pattern.dtype)[...] = pattern
    return k, v


def scatter(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
            slots: np.ndarray) -> None:
    """Write token i's K/V ``[H_kv][d]`` into slot ``slots[i]``; slot -1 means skip.

    This is the "write the new token's K/V into its slot" step that decoding
    implies: only the new token's key and value are computed, the rest is read
    back from the cache ([P4] KV-cache introduction; [P2] core idea item 3).
    """
    nb, H, npieces, B, X = k_cache.shape
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    if np.any(slots[keep] >= nb * B):
        raise ValueError("slot out of range")
    if len(np.unique(slots[keep])) != int(keep.sum()):
        raise ValueError("duplicate slot in one scatter")
    s = slots[keep]
    blk, off = s // B, s % B
    kn = np.asarray(k_new)[keep]
    vn = np.asarray(v_new)[keep]
    k_cache[blk, :, :, off, :] = kn.reshape(len(s), H, npieces, X)
    v_cache[blk, :, :, off] = vn


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs: np.ndarray) -> None:
    """Copy whole blocks (all heads, all slots) ``src -> dst`` for each pair, in order.

    The device side of copy-on-write: a branch about to write into a shared,
    not-full block gets its own copy first ([P3] section 3; [P2] key technical
    point 3).
    """
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray, pairs) -> None:
    """Copy whole blocks from one cache pair to another: dst block j <- src block i for each (i, j).

    The data half of preemption by swapping: a waiting sequence's blocks move
    to host memory and later back ([P2] section 4; [P4] "Preemption").
    """
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]


def gather(k_cache: np.ndarray, v_cache: np.ndarray, table, n: int) -> Tuple[np.ndarray, np.ndarray]:
    """Logical K and V ``[n][H_kv][d]`` of a sequence, read through its block table."""
    nb, H, npieces, B, X = k_cache.shape
    t = np.arange(n)
    blk = np.asarray(table, dtype=np.int64)[t // B]
    if np.any(blk < 0) or np.any(blk >= nb):
        raise ValueError("block table entry out of range")
    off = t % B
    k = k_cache[blk, :, :, off, :].reshape(n, H, npieces * X)
    v = v_cache[blk, :, :, off]
    return k, v


def to_f64(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Exact widening of stored values (float32, or bfloat16 bits in uint16) to float64."""
    if kv_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(kv_dtype)
