"""paged_kv_cache_physical_amd — Python binding of libpkv, the paged KV-cache
attention path for AMD MI355X (gfx950): a host block pool (refcounted sharing,
copy-on-write, swapping, prefix caching, rollback), decode attention, runs of
causal queries (prefill, prefix-cached tails, speculative verification) and the
cache writes and block copies around them.

Argument marshalling only: every call below forwards to the C function of the
same name in ``libpkv.so`` (declared in ``include/pkv.h``); host arrays are
NumPy, device buffers are torch tensors (PyTorch provides device memory and
streams, nothing else).  The library must have been built first
(``python -m paged_kv_cache_physical_amd.build``); otherwise every call raises.

Cache tensors use the interface's physical layout:
  key cache    [num_blocks][H_kv][d / X][B][X],  X = 16 / bytes_per_scalar
  value cache  [num_blocks][H_kv][d][B]
Host caches for swapping have the same layout in page-locked host memory.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from ._lib import (PKV_BF16, PKV_ERR_INVALID_ARG, PKV_F32, InvalidArg, NoSuchSeq, OutOfBlocks, PkvError, Stats, WrongTier,  # noqa: F401
                   check, header_symbols, lib)

__all__ = [
    "pkv_pool_create", "pkv_pool_destroy", "pkv_seq_create", "pkv_seq_fork", "pkv_seq_free", "pkv_append_tokens",
    "pkv_seq_create_prefixed", "pkv_pool_cached_blocks", "pkv_seq_truncate", "pkv_paged_attention_multi",
    "pkv_attention_multi_workspace_bytes",
    "pkv_block_tables", "pkv_seq_info", "pkv_pool_stats", "pkv_block_refcount", "pkv_pool_free_list",
    "pkv_pool_validate", "pkv_pool_set_host_blocks", "pkv_swap_out", "pkv_swap_in", "pkv_seq_table",
    "pkv_host_block_refcount", "pkv_pool_host_free_list", "pkv_swap_blocks", "empty_host_caches", "pkv_reshape_and_cache", "pkv_copy_blocks", "pkv_attention_workspace_bytes",
    "pkv_paged_attention_decode", "pkv_paged_attention_partitions", "pkv_paged_attention_reduce",
    "pkv_decode_step", "pkv_decode_step_static", "pkv_abi_version", "pkv_hbm_read_probe", "Pool", "cache_shapes", "empty_caches", "PkvError",
    "OutOfBlocks", "NoSuchSeq", "InvalidArg", "WrongTier",
]


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None and a.size else None


def pkv_abi_version() -> int:
    return int(lib().pkv_abi_version())


# ---------------------------------------------------------------------------
# Host block pool
# ---------------------------------------------------------------------------


def pkv_pool_create(num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None) -> ctypes.c_void_p:
    order = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
    if order is not None and order.size != num_blocks:
        raise InvalidArg(-1, "pkv_pool_create", "free_order length differs from num_blocks")
    out = ctypes.c_void_p()
    check(lib().pkv_pool_create(num_blocks, block_size, _ptr(order), ctypes.byref(out)), "pkv_pool_create")
    return out


def pkv_pool_destroy(pool) -> None:
    lib().pkv_pool_destroy(pool)


def pkv_seq_create(pool) -> int:
    sid = ctypes.c_int32()
    check(lib().pkv_seq_create(pool, ctypes.byref(sid)), "pkv_seq_create")
    return sid.value


def pkv_seq_fork(pool, parent: int) -> int:
    sid = ctypes.c_int32()
    check(lib().pkv_seq_fork(pool, parent, ctypes.byref(sid)), "pkv_seq_fork")
    return sid.value


def pkv_seq_free(pool, seq: int) -> None:
    check(lib().pkv_seq_free(pool, seq), "pkv_seq_free")


def pkv_append_tokens(pool, seqs: Sequence[int], counts: Sequence[int],
                      token_ids: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Returns (slots int64[sum counts], copy-on-write pairs int32[k][2]); token_ids (one per new token,
    sequence-major) keys the blocks the batch fills for prefix caching."""
    seqs = np.ascontiguousarray(seqs, dtype=np.int32)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    if seqs.shape != counts.shape or seqs.ndim != 1:
        raise InvalidArg(-1, "pkv_append_tokens", "seqs and counts must be 1-D and equal in length")
    total = int(counts[counts > 0].sum()) if counts.size else 0
    ids = None
    if token_ids is not None:
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
        if ids.ndim != 1 or ids.size != total:
            raise InvalidArg(-1, "pkv_append_tokens", "one token id per appended token")
    slots = np.empty(max(total, 0), dtype=np.int64)
    pairs = np.empty((max(len(seqs), 1), 2), dtype=np.int32)
    n_cow = ctypes.c_int32()
    # an empty id list is still "ids given": pass a valid pointer
    ids_ptr = None if ids is None else ids.ctypes.data_as(ctypes.c_void_p) if ids.size else \
        np.zeros(1, dtype=np.int32).ctypes.data_as(ctypes.c_void_p)
    check(lib().pkv_append_tokens(pool, _ptr(seqs), _ptr(counts), len(seqs), ids_ptr, _ptr(slots), slots.size,
                                  _ptr(pairs), pairs.shape[0], ctypes.byref(n_cow)), "pkv_append_tokens")
    return slots, pairs[:n_cow.value].copy()


def pkv_seq_truncate(pool, seq: int, new_len: int) -> None:
    check(lib().pkv_seq_truncate(pool, seq, new_len), "pkv_seq_truncate")


def pkv_seq_create_prefixed(pool, token_ids: Sequence[int]) -> Tuple[int, int]:
    """New sequence for a prompt: maps its longest run of cached leading blocks; returns (seq, cached tokens)."""
    ids = np.ascontiguousarray(token_ids, dtype=np.int32)
    if ids.ndim != 1:
        raise InvalidArg(-1, "pkv_seq_create_prefixed", "token_ids must be 1-D")
    sid, hit = ctypes.c_int32(), ctypes.c_int32()
    check(lib().pkv_seq_create_prefixed(pool, _ptr(ids), ids.size, ctypes.byref(sid), ctypes.byref(hit)),
          "pkv_seq_create_prefixed")
    return sid.value, hit.value


def pkv_pool_cached_blocks(pool) -> dict:
    """The prefix cache: {key: device block}."""
    n = ctypes.c_int32()
    lib().pkv_pool_cached_blocks(pool, None, None, 0, ctypes.byref(n))
    keys = np.empty(n.value, dtype=np.uint64)
    blocks = np.empty(n.value, dtype=np.int32)
    check(lib().pkv_pool_cached_blocks(pool, _ptr(keys), _ptr(blocks), n.value, ctypes.byref(n)),
          "pkv_pool_cached_blocks")
    return {int(k): int(b) for k, b in zip(keys, blocks)}


def pkv_block_tables(pool, seqs: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
    seqs = np.ascontiguousarray(seqs, dtype=np.int32)
    tables = np.empty((len(seqs), max_blocks), dtype=np.int32)
    lens = np.empty(len(seqs), dtype=np.int32)
    check(lib().pkv_block_tables(pool, _ptr(seqs), len(seqs), max_blocks, _ptr(tables), _ptr(lens)),
          "pkv_block_tables")
    return tables, lens


def pkv_seq_info(pool, seq: int) -> Tuple[int, int]:
    n, nb = ctypes.c_int32(), ctypes.c_int32()
    check(lib().pkv_seq_info(pool, seq, ctypes.byref(n), ctypes.byref(nb)), "pkv_seq_info")
    return n.value, nb.value


def pkv_pool_stats(pool) -> dict:
    st = Stats()
    check(lib().pkv_pool_stats(pool, ctypes.byref(st)), "pkv_pool_stats")
    return st.as_dict()


def pkv_block_refcount(pool, block: int) -> int:
    return int(lib().pkv_block_refcount(pool, block))


def _free_list(fn, name, pool) -> np.ndarray:
    n = ctypes.c_int32()
    fn(pool, None, 0, ctypes.byref(n))
    out = np.empty(n.value, dtype=np.int32)
    check(fn(pool, _ptr(out), out.size, ctypes.byref(n)), name)
    return out


def pkv_pool_free_list(pool) -> np.ndarray:
    return _free_list(lib().pkv_pool_free_list, "pkv_pool_free_list", pool)


def pkv_pool_host_free_list(pool) -> np.ndarray:
    return _free_list(lib().pkv_pool_host_free_list, "pkv_pool_host_free_list", pool)


def pkv_pool_set_host_blocks(pool, num_host_blocks: int) -> None:
    check(lib().pkv_pool_set_host_blocks(pool, num_host_blocks), "pkv_pool_set_host_blocks")


def _swap(fn, name, pool, seqs) -> np.ndarray:
    seqs = np.ascontiguousarray(seqs, dtype=np.int32)
    if seqs.ndim != 1:
        raise InvalidArg(-1, name, "seqs must be 1-D")
    n = ctypes.c_int32()
    pairs = np.empty((64, 2), dtype=np.int32)
    st = fn(pool, _ptr(seqs), len(seqs), _ptr(pairs), pairs.shape[0], ctypes.byref(n))
    if st == PKV_ERR_INVALID_ARG and n.value > pairs.shape[0]:  # more pairs than the first guess: make room
        pairs = np.empty((n.value, 2), dtype=np.int32)
        st = fn(pool, _ptr(seqs), len(seqs), _ptr(pairs), pairs.shape[0], ctypes.byref(n))
    check(st, name)
    return pairs[:n.value].copy()


def pkv_swap_out(pool, seqs: Sequence[int]) -> np.ndarray:
    """Move a whole sharing group to the host tier; returns (device block, host block) pairs."""
    return _swap(lib().pkv_swap_out, "pkv_swap_out", pool, seqs)


def pkv_swap_in(pool, seqs: Sequence[int]) -> np.ndarray:
    """Bring swapped-out sequences back; returns (host block, device block) pairs."""
    return _swap(lib().pkv_swap_in, "pkv_swap_in", pool, seqs)


def pkv_seq_table(pool, seq: int) -> Tuple[np.ndarray, bool]:
    """One sequence's block ids in its current tier, and whether it is swapped out."""
    n, host = ctypes.c_int32(), ctypes.c_int32()
    lib().pkv_seq_table(pool, seq, None, 0, ctypes.byref(n), ctypes.byref(host))
    out = np.empty(n.value, dtype=np.int32)
    check(lib().pkv_seq_table(pool, seq, _ptr(out), out.size, ctypes.byref(n), ctypes.byref(host)), "pkv_seq_table")
    return out, bool(host.value)


def pkv_host_block_refcount(pool, block: int) -> int:
    return int(lib().pkv_host_block_refcount(pool, block))


def pkv_pool_validate(pool) -> None:
    check(lib().pkv_pool_validate(pool), "pkv_pool_validate")


class Pool:
    """Owning wrapper around a pkv_pool handle; methods map 1:1 onto the C calls."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None, host_blocks: int = 0):
        self.handle = pkv_pool_create(num_blocks, block_size, free_order)
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.host_blocks = host_blocks
        if host_blocks:
            pkv_pool_set_host_blocks(self.handle, host_blocks)

    def close(self):
        if self.handle is not None:
            pkv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def create(self) -> int:
        return pkv_seq_create(self.handle)

    def fork(self, parent: int) -> int:
        return pkv_seq_fork(self.handle, parent)

    def free_seq(self, seq: int) -> None:
        pkv_seq_free(self.handle, seq)

    def append(self, seqs, counts, token_ids=None):
        return pkv_append_tokens(self.handle, seqs, counts, token_ids)

    def truncate(self, seq: int, new_len: int) -> None:
        pkv_seq_truncate(self.handle, seq, new_len)

    def length(self, seq: int) -> int:
        return self.info(seq)[0]

    def create_prefixed(self, token_ids):
        return pkv_seq_create_prefixed(self.handle, token_ids)

    def cached(self) -> dict:
        return pkv_pool_cached_blocks(self.handle)

    def block_tables(self, seqs, max_blocks):
        return pkv_block_tables(self.handle, seqs, max_blocks)

    def info(self, seq):
        return pkv_seq_info(self.handle, seq)

    def stats(self) -> dict:
        return pkv_pool_stats(self.handle)

    def refcount(self, block: int) -> int:
        return pkv_block_refcount(self.handle, block)

    def free_list(self) -> np.ndarray:
        return pkv_pool_free_list(self.handle)

    def validate(self) -> None:
        pkv_pool_validate(self.handle)

    def swap_out(self, seqs) -> np.ndarray:
        return pkv_swap_out(self.handle, seqs)

    def swap_in(self, seqs) -> np.ndarray:
        return pkv_swap_in(self.handle, seqs)

    def table(self, seq: int) -> np.ndarray:
        return pkv_seq_table(self.handle, seq)[0]

    def on_host(self, seq: int) -> bool:
        return pkv_seq_table(self.handle, seq)[1]

    def host_refcount(self, block: int) -> int:
        return pkv_host_block_refcount(self.handle, block)

    def host_free_list(self) -> np.ndarray:
        return pkv_pool_host_free_list(self.handle)


# ---------------------------------------------------------------------------
# Device calls (torch tensors on the GPU)
# ---------------------------------------------------------------------------


def _torch():
    import torch
    return torch


def _dtype_name(t) -> str:
    return "f32" if _dtype_code(t) == PKV_F32 else "bf16"


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise InvalidArg(-1, "dtype", f"unsupported tensor dtype {t.dtype}")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise InvalidArg(-1, name, "tensor must be on the GPU")
    if not t.is_contiguous():
        raise InvalidArg(-1, name, "tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def cache_shapes(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, kv_dtype: str):
    X = 16 // (4 if kv_dtype == "f32" else 2)
    return ((num_blocks, num_kv_heads, head_dim // X, block_size, X), (num_blocks, num_kv_heads, head_dim, block_size))


def empty_caches(num_blocks, num_kv_heads, block_size, head_dim, kv_dtype: str, device="cuda", poison=True):
    """Key/value cache tensors in the interface layout, optionally filled with NaN."""
    torch = _torch()
    dt = torch.float32 if kv_dtype == "f32" else torch.bfloat16
    ks, vs = cache_shapes(num_blocks, num_kv_heads, block_size, head_dim, kv_dtype)
    k = torch.empty(ks, dtype=dt, device=device)
    v = torch.empty(vs, dtype=dt, device=device)
    if poison:
        if kv_dtype == "f32":
            k.view(torch.int32).fill_(0x7FC00000)
            v.view(torch.int32).fill_(0x7FC00000)
        else:
            k.view(torch.int16).fill_(0x7FC0)
            v.view(torch.int16).fill_(0x7FC0)
    return k, v


def empty_host_caches(num_blocks, num_kv_heads, block_size, head_dim, kv_dtype: str):
    """Key/value caches of the host tier: the interface layout in page-locked host memory."""
    torch = _torch()
    dt = torch.float32 if kv_dtype == "f32" else torch.bfloat16
    ks, vs = cache_shapes(num_blocks, num_kv_heads, block_size, head_dim, kv_dtype)
    return torch.empty(ks, dtype=dt, pin_memory=True), torch.empty(vs, dtype=dt, pin_memory=True)


def _reachable(t, name):
    """A tensor the GPU can reach: on the GPU, or in page-locked host memory."""
    if not (t.is_cuda or t.is_pinned()):
        raise InvalidArg(-1, name, "tensor must be on the GPU or in page-locked host memory")
    if not t.is_contiguous():
        raise InvalidArg(-1, name, "tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def pkv_swap_blocks(src_k, src_v, dst_k, dst_v, pairs, stream=None) -> None:
    """Copy blocks src -> dst for each (src block, dst block) in pairs (int32[n][2], GPU or pinned); the caches
    are device or page-locked host tensors of one layout (the pairs of pkv_swap_out / pkv_swap_in)."""
    torch = _torch()
    if pairs.dtype != torch.int32 or (pairs.numel() and (pairs.dim() != 2 or pairs.shape[1] != 2)):
        raise InvalidArg(-1, "pkv_swap_blocks", "pairs must be int32[n][2]")
    if src_k.shape[1:] != dst_k.shape[1:] or src_v.shape[1:] != dst_v.shape[1:] or \
            src_k.shape[0] != src_v.shape[0] or dst_k.shape[0] != dst_v.shape[0] or \
            len({src_k.dtype, src_v.dtype, dst_k.dtype, dst_v.dtype}) != 1 or src_k[0].numel() != src_v[0].numel():
        raise InvalidArg(-1, "pkv_swap_blocks", "the caches must share a block layout and dtype")
    n = pairs.shape[0] if pairs.numel() else 0
    if n == 0:
        return
    block_bytes = src_k[0].numel() * src_k.element_size()
    check(lib().pkv_swap_blocks(_reachable(src_k, "src_k"), _reachable(src_v, "src_v"), _reachable(dst_k, "dst_k"),
                                _reachable(dst_v, "dst_v"), _reachable(pairs, "pairs"), n, src_k.shape[0],
                                dst_k.shape[0], block_bytes, _stream(stream)), "pkv_swap_blocks")


def pkv_reshape_and_cache(k_new, v_new, k_cache, v_cache, slots, block_size: int, stream=None) -> None:
    """k_new, v_new: [T][H_kv][d]; slots: int64[T] on the GPU."""
    if k_new.dim() != 3 or k_new.shape != v_new.shape:
        raise InvalidArg(-1, "pkv_reshape_and_cache", "k_new and v_new must be [T][H_kv][d] and equal")
    T, H, d = k_new.shape
    torch = _torch()
    if slots.dtype != torch.int64 or slots.numel() != T:
        raise InvalidArg(-1, "pkv_reshape_and_cache", "slots must be int64[T]")
    for t in (v_new, k_cache, v_cache):
        if t.dtype != k_new.dtype:
            raise InvalidArg(-1, "pkv_reshape_and_cache", "dtype mismatch")
    nb = v_cache.shape[0]
    ks, vs = cache_shapes(nb, H, block_size, d, _dtype_name(k_new))
    if tuple(k_cache.shape) != ks or tuple(v_cache.shape) != vs:
        raise InvalidArg(-1, "pkv_reshape_and_cache", "cache shape does not match k_new / block_size")
    check(lib().pkv_reshape_and_cache(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"),
                                      _dev(v_cache, "v_cache"), _dev(slots, "slots"), T, H, d, block_size, nb,
                                      _dtype_code(k_new), _stream(stream)), "pkv_reshape_and_cache")


def pkv_copy_blocks(k_cache, v_cache, pairs, stream=None) -> None:
    """pairs: int32[n][2] (src, dst) on the GPU."""
    torch = _torch()
    if pairs.dtype != torch.int32 or (pairs.numel() and (pairs.dim() != 2 or pairs.shape[1] != 2)):
        raise InvalidArg(-1, "pkv_copy_blocks", "pairs must be int32[n][2]")
    n = pairs.shape[0] if pairs.numel() else 0
    if n == 0:
        return
    nb = v_cache.shape[0]
    block_bytes = v_cache[0].numel() * v_cache.element_size()
    check(lib().pkv_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(pairs, "pairs"), n, nb,
                                block_bytes, _stream(stream)), "pkv_copy_blocks")


def pkv_hbm_read_probe(buf, sink, stream=None) -> None:
    """Stream-read the whole of `buf` (a GPU tensor); `sink` is an int32/uint32 GPU tensor of >= 1 element."""
    nbytes = buf.numel() * buf.element_size()
    check(lib().pkv_hbm_read_probe(_dev(buf, "buf"), nbytes, _dev(sink, "sink"), _stream(stream)),
          "pkv_hbm_read_probe")


def pkv_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                                  partition_size) -> int:
    return int(lib().pkv_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                                   max_context_len, partition_size))


def _attention(fn: str, out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int, scale: float,
               partition_size: int = 0, workspace=None, stream=None, new_kv=None, static_scratch=False) -> None:
    torch = _torch()
    S, Hq, d = q.shape
    nb, Hkv, d2, B = v_cache.shape
    if d2 != d or out.shape != q.shape or out.dtype != torch.float32:
        raise InvalidArg(-1, fn, "shape mismatch")
    if tuple(k_cache.shape) != cache_shapes(nb, Hkv, B, d, _dtype_name(q))[0]:
        raise InvalidArg(-1, fn, "key cache shape mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise InvalidArg(-1, fn, "tables and lengths must be int32")
    if block_tables.shape[0] != S or context_lens.numel() != S or q.dtype != k_cache.dtype:
        raise InvalidArg(-1, fn, "shape or dtype mismatch")
    max_blocks = block_tables.shape[1]
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    lead = []
    if new_kv is not None:
        k_new, v_new = new_kv
        if tuple(k_new.shape) != (S, Hkv, d) or tuple(v_new.shape) != (S, Hkv, d) or \
                k_new.dtype != q.dtype or v_new.dtype != q.dtype:
            raise InvalidArg(-1, fn, "new token shape or dtype mismatch")
        lead = [_dev(k_new, "k_new"), _dev(v_new, "v_new")]
    ws_args = [] if static_scratch else [ws_ptr, ws_bytes]
    check(getattr(lib(), fn)(*lead, _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"),
                             _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
                             _dev(context_lens, "context_lens"), S, Hq, Hkv, d, B, nb, max_blocks,
                             int(max_context_len), float(scale), int(partition_size), *ws_args,
                             _dtype_code(q), _stream(stream)), fn)


def pkv_paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                               scale: float, partition_size: int = 0, workspace=None, stream=None) -> None:
    """out: fp32 [S][H_q][d]; q: [S][H_q][d] (cache dtype); block_tables int32 [S][max_blocks];
    context_lens int32 [S]; workspace: uint8 tensor of >= pkv_attention_workspace_bytes(...) bytes."""
    _attention("pkv_paged_attention_decode", out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
               scale, partition_size, workspace, stream)


def pkv_decode_step(k_new, v_new, out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                    scale: float, partition_size: int = 0, workspace=None, stream=None) -> None:
    """One decode step: write k_new, v_new ([S][H_kv][d], cache dtype; the token at position n_s - 1 of each
    sequence) into the caches through the block tables, then pkv_paged_attention_decode (same arguments)."""
    _attention("pkv_decode_step", out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
               partition_size, workspace, stream, new_kv=(k_new, v_new))


def pkv_decode_step_static(k_new, v_new, out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                           scale: float, partition_size: int = 0, stream=None) -> None:
    """pkv_decode_step with the library's static device scratch instead of a workspace (for callers that cannot
    allocate); calls that overlap on one GPU race."""
    _attention("pkv_decode_step_static", out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
               scale, partition_size, None, stream, new_kv=(k_new, v_new), static_scratch=True)


def pkv_attention_multi_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                        max_query_len) -> int:
    return int(lib().pkv_attention_multi_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                         max_context_len, max_query_len))


def pkv_paged_attention_multi(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                              max_context_len: int, max_query_len: int, scale: float, stream=None,
                              workspace=None, seq_order=None) -> None:
    """Runs of causal queries: out fp32 [T][H_q][d]; q [T][H_q][d] (cache dtype); query_start int32 [S+1]
    (rows of sequence s: its last query_start[s+1] - query_start[s] positions); block_tables int32
    [S][max_blocks]; context_lens int32 [S]; workspace: uint8 tensor of >= pkv_attention_multi_workspace_bytes
    bytes, or None (no context split); seq_order: int32 [S] on the GPU, the order to start the sequences in
    (e.g. longest first), or None."""
    torch = _torch()
    fn = "pkv_paged_attention_multi"
    if q.dim() != 3 or out.shape != q.shape or out.dtype != torch.float32:
        raise InvalidArg(-1, fn, "out and q must be [T][H_q][d], out fp32")
    T, Hq, d = q.shape
    nb, Hkv, d2, B = v_cache.shape
    if d2 != d or q.dtype != k_cache.dtype or q.dtype != v_cache.dtype:
        raise InvalidArg(-1, fn, "q and caches disagree in d or dtype")
    ks, vs = cache_shapes(nb, Hkv, B, d, _dtype_name(q))
    if tuple(k_cache.shape) != ks:
        raise InvalidArg(-1, fn, "key cache shape")
    S = context_lens.numel()
    for t, name, shape in ((block_tables, "block_tables", None), (context_lens, "context_lens", (S,)),
                           (query_start, "query_start", (S + 1,))):
        if t.dtype != torch.int32 or (shape is not None and tuple(t.shape) != shape):
            raise InvalidArg(-1, fn, f"{name} must be int32" + (f" of shape {shape}" if shape else ""))
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise InvalidArg(-1, fn, "block_tables must be [S][max_blocks]")
    if seq_order is not None and (seq_order.dtype != torch.int32 or tuple(seq_order.shape) != (S,)):
        raise InvalidArg(-1, fn, "seq_order must be int32 [S]")
    check(lib().pkv_paged_attention_multi(_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"),
                                          _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
                                          _dev(context_lens, "context_lens"), _dev(query_start, "query_start"),
                                          None if seq_order is None else _dev(seq_order, "seq_order"), S, T,
                                          Hq, Hkv, d, B, nb, block_tables.shape[1], max_context_len, max_query_len,
                                          scale, None if workspace is None else _dev(workspace, "workspace"),
                                          0 if workspace is None else workspace.numel() * workspace.element_size(),
                                          _dtype_code(q), _stream(stream)), fn)


def pkv_paged_attention_partitions(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                                   scale: float, partition_size: int = 0, workspace=None, stream=None) -> None:
    """First stage of pkv_paged_attention_decode (same arguments)."""
    _attention("pkv_paged_attention_partitions", out, q, k_cache, v_cache, block_tables, context_lens,
               max_context_len, scale, partition_size, workspace, stream)


def pkv_paged_attention_reduce(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                               scale: float, partition_size: int = 0, workspace=None, stream=None) -> None:
    """Second stage of pkv_paged_attention_decode (same arguments)."""
    _attention("pkv_paged_attention_reduce", out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
               scale, partition_size, workspace, stream)
