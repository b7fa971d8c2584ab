"""Drive one decode batch through libpkv: replay a workload's allocator script with
the C pool, apply its block copies and K/V writes with the HIP kernels, and run
decode attention.  Used by the tests, the smoke check and the benchmark."""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from . import (Pool, empty_caches, pkv_attention_workspace_bytes, pkv_copy_blocks, pkv_decode_step,
               pkv_paged_attention_decode,
               pkv_paged_attention_partitions, pkv_paged_attention_reduce, pkv_reshape_and_cache)


def _to_device(arr: np.ndarray, kv_dtype: str, device):
    import torch
    if kv_dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16)).to(device).view(torch.bfloat16)


@dataclass
class DecodeInputs:
    k_new: object
    v_new: object
    slots: object


class GpuBatch:
    """Device state of one workload after its script has run (the decode token included)."""

    def __init__(self, workload, device="cuda", poison: bool = True, pool: Optional[Pool] = None):
        import torch

        s = workload.spec
        self.workload = workload
        self.device = device
        self.pool = pool or Pool(workload.num_blocks, s.block_size, workload.free_order)
        self.k_cache, self.v_cache = empty_caches(workload.num_blocks, s.num_kv_heads, s.block_size, s.head_dim,
                                                  s.kv_dtype, device=device, poison=poison)
        self.seq_ids: List[int] = []
        self.slots: List[np.ndarray] = []
        self.pairs: List[np.ndarray] = []
        self.decode: Optional[DecodeInputs] = None
        from workloads import Append, Create, Fork  # input structure only

        for op in workload.script():
            if isinstance(op, Create):
                self.seq_ids.extend(self.pool.create() for _ in range(op.count))
            elif isinstance(op, Fork):
                self.seq_ids.append(self.pool.fork(op.parent))
            elif isinstance(op, Append):
                slots, pairs = self.pool.append(op.seqs, op.counts)
                self.slots.append(slots)
                self.pairs.append(pairs)
                if len(pairs):
                    pkv_copy_blocks(self.k_cache, self.v_cache, torch.from_numpy(pairs).to(device))
                if len(slots):
                    k, v = op.values()
                    kd, vd = _to_device(k, s.kv_dtype, device), _to_device(v, s.kv_dtype, device)
                    sd = torch.from_numpy(slots).to(device)
                    pkv_reshape_and_cache(kd, vd, self.k_cache, self.v_cache, sd, s.block_size)
                    if op.decode:
                        self.decode = DecodeInputs(kd, vd, sd)
                        decode_seqs = np.asarray(op.seqs)
                    del k, v
            else:
                raise TypeError(op)
        ids = sorted(self.seq_ids)
        # pkv_decode_step pairs row i of the new K/V with row i of the block table
        self.decode_rows_match = self.decode is not None and np.array_equal(decode_seqs, np.asarray(ids))
        self.max_blocks = max(1, max(self.pool.info(i)[1] for i in ids)) if ids else 1
        tables, lens = self.pool.block_tables(ids, self.max_blocks)
        self.tables_host, self.lens_host = tables, lens
        self.block_tables = torch.from_numpy(tables).to(device)
        self.context_lens = torch.from_numpy(lens).to(device)
        self.max_context_len = int(lens.max()) if len(lens) else 0
        self.q = _to_device(workload.q, s.kv_dtype, device)
        self.out = torch.empty(self.q.shape, dtype=torch.float32, device=device)
        self._ws = {}
        torch.cuda.synchronize()

    def workspace(self, partition_size: int):
        import torch
        s = self.workload.spec
        nbytes = pkv_attention_workspace_bytes(self.q.shape[0], s.num_q_heads, s.num_kv_heads, s.head_dim,
                                               s.block_size, self.max_context_len, partition_size)
        if nbytes == 0:
            return None
        ws = self._ws.get(nbytes)
        if ws is None:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._ws[nbytes] = ws
        return ws

    def attention(self, partition_size: Optional[int] = None, out=None, stream=None):
        p = self.workload.spec.partition_size if partition_size is None else partition_size
        out = self.out if out is None else out
        pkv_paged_attention_decode(out, self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                                   self.max_context_len, float(self.workload.scale), p, self.workspace(p), stream)
        return out

    def _args(self, partition_size):
        p = self.workload.spec.partition_size if partition_size is None else partition_size
        return (self.out, self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                self.max_context_len, float(self.workload.scale), p, self.workspace(p))

    def attention_partitions(self, partition_size: Optional[int] = None, stream=None):
        pkv_paged_attention_partitions(*self._args(partition_size), stream)

    def attention_reduce(self, partition_size: Optional[int] = None, stream=None):
        pkv_paged_attention_reduce(*self._args(partition_size), stream)

    def write_decode_token(self, stream=None):
        """Re-issue the decode step's K/V write (idempotent: same slots, same values)."""
        d = self.decode
        pkv_reshape_and_cache(d.k_new, d.v_new, self.k_cache, self.v_cache, d.slots,
                              self.workload.spec.block_size, stream)

    def step(self, partition_size: Optional[int] = None, stream=None):
        """One decode step: write each sequence's new token, then attend over its context (one call)."""
        p = self.workload.spec.partition_size if partition_size is None else partition_size
        d = self.decode
        if not self.decode_rows_match:
            raise ValueError("the decode token rows are not in block-table row order")
        pkv_decode_step(d.k_new, d.v_new, self.out, self.q, self.k_cache, self.v_cache, self.block_tables,
                        self.context_lens, self.max_context_len, float(self.workload.scale), p, self.workspace(p),
                        stream)
        return self.out

    def step_separate(self, partition_size: Optional[int] = None, stream=None):
        """The same step as two calls: pkv_reshape_and_cache, then pkv_paged_attention_decode."""
        self.write_decode_token(stream)
        return self.attention(partition_size, stream=stream)
