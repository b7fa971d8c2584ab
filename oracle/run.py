"""Replay a workload's allocator script with the oracle's own pieces (test infrastructure).

Each ``Append`` asks the oracle allocator for slots and copy-on-write pairs,
applies the block copies, then scatters the tokens' K/V, in that order: a
branch's shared partial block is copied before anything is written into it
([P3] section 3).  The result is the expected state of every device buffer.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from . import allocator as _alloc
from . import cache as _cache


@dataclass
class Replay:
    pool: _alloc.BlockPool
    k_cache: np.ndarray
    v_cache: np.ndarray
    seq_ids: List[int]
    slots: List[np.ndarray] = field(default_factory=list)  # per Append op
    pairs: List[np.ndarray] = field(default_factory=list)  # per Append op
    tables: np.ndarray = None
    context_lens: np.ndarray = None
    max_blocks: int = 0


def replay(workload, with_cache: bool = True, host_blocks: int = 0) -> Replay:
    """Run ``workload.script()``; with ``with_cache=False`` only the allocator is replayed.  ``host_blocks``
    gives the pool a host tier for later swaps."""
    from workloads import Append, Create, Fork  # input structure only

    s = workload.spec
    pool = _alloc.BlockPool(workload.num_blocks, s.block_size, workload.free_order, host_blocks=host_blocks)
    if with_cache:
        kc, vc = _cache.empty_caches(workload.num_blocks, s.num_kv_heads, s.block_size, s.head_dim, s.kv_dtype)
    else:
        kc = vc = None
    rp = Replay(pool, kc, vc, [])
    for op in workload.script():
        if isinstance(op, Create):
            rp.seq_ids.extend(pool.create() for _ in range(op.count))
        elif isinstance(op, Fork):
            rp.seq_ids.append(pool.fork(op.parent))
        elif isinstance(op, Append):
            slots, pairs = pool.append(op.seqs, op.counts)
            rp.slots.append(slots)
            rp.pairs.append(pairs)
            if with_cache:
                _cache.copy_blocks(kc, vc, pairs)
                k, v = op.values()
                _cache.scatter(kc, vc, k, v, slots)
        else:
            raise TypeError(op)
    ids = sorted(rp.seq_ids)
    rp.max_blocks = max((len(pool.table(i)) for i in ids), default=0)
    rp.tables, rp.context_lens = pool.block_tables(ids, max(rp.max_blocks, 1))
    return rp
