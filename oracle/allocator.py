"""Block-pool model with refcounts and copy-on-write (test infrastructure; see oracle/__init__).

What it follows:
  * Fixed-size blocks, a per-sequence block table mapping logical block i to a
    physical block, allocation only when a sequence grows onto a new block
    ([P2] "core idea" items 1-4; [P1] summary "on-demand allocation").
  * A finished request's blocks return to the pool at once ([P2] key
    technical point 2; [P3] section 3: cancel/timeout also reclaim).
  * Several sequences may map logical blocks to one physical block; a shared
    count tied to request lifetime; a branch that writes into a shared block
    that is not yet full copies it first ([P3] section 3; [P4] beam-search
    sharing figure; [P2] key technical point 3).

Readings where the pages are silent:
  * The free blocks form a FIFO queue seeded by a given order: allocation pops
    the head, a freed block joins the tail.
  * Copy-on-write fires on append when the sequence's last block is partly
    filled and its refcount exceeds 1: a fresh block is popped, the pair
    (old, new) is reported for the device copy, the old block's count drops by
    one and the table points at the new block.  The last holder (count 1)
    writes in place; full blocks are never written again and so never copied.
  * An append batch is all or nothing: if the pool runs out, nothing changes.
  * Token position p of a sequence lives in slot table[p // B] * B + p % B.

This model applies each batch to a deep copy of the state and commits the copy
only on success, which makes the all-or-nothing rule evident.
"""

from __future__ import annotations

import copy
from collections import deque
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


class PoolError(Exception):
    pass


class OutOfBlocks(PoolError):
    pass


class NoSuchSeq(PoolError):
    pass


class InvalidArg(PoolError):
    pass


@dataclass
class _Seq:
    table: List[int] = field(default_factory=list)
    length: int = 0


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidArg("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: deque = deque(order)
        self.refcount = [0] * num_blocks
        self.seqs: Dict[int, _Seq] = {}
        self.next_id = 0

    # -- sequences -----------------------------------------------------------
    def create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = _Seq()
        return sid

    def _get(self, sid: int) -> _Seq:
        if sid not in self.seqs:
            raise NoSuchSeq(sid)
        return self.seqs[sid]

    def fork(self, parent: int) -> int:
        """New sequence sharing every block of ``parent``; each shared block's count rises by one."""
        p = self._get(parent)
        sid = self.create()
        self.seqs[sid] = _Seq(table=list(p.table), length=p.length)
        for b in p.table:
            self.refcount[b] += 1
        return sid

    def free_seq(self, sid: int) -> None:
        """Release ``sid``: counts drop in logical order; blocks reaching zero join the queue's tail."""
        s = self._get(sid)
        for b in s.table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.seqs[sid]

    # -- appends ---------------------------------------------------------------
    def _pop(self) -> int:
        if not self.free:
            raise OutOfBlocks()
        b = self.free.popleft()
        self.refcount[b] = 1
        return b

    def _append_one(self, sid: int, count: int, slots: List[int], pairs: List[Tuple[int, int]]) -> None:
        B = self.block_size
        s = self._get(sid)
        if count == 0:
            return
        if s.length % B != 0:
            last = s.table[-1]
            if self.refcount[last] > 1:
                new = self._pop()
                pairs.append((last, new))
                self.refcount[last] -= 1
                s.table[-1] = new
        for p in range(s.length, s.length + count):
            if p % B == 0:
                s.table.append(self._pop())
            slots.append(s.table[p // B] * B + p % B)
        s.length += count

    def append(self, seqs: Sequence[int], counts: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
        """Append ``counts[i]`` tokens to ``seqs[i]``, in order; all or nothing.

        Returns ``(slots int64[sum counts], pairs int32[k][2])``; slots are in
        sequence-major, position order.  Raises OutOfBlocks (state unchanged)
        when the pool cannot hold the whole batch.
        """
        seqs = [int(x) for x in seqs]
        counts = [int(c) for c in counts]
        if len(seqs) != len(counts):
            raise InvalidArg("seqs and counts differ in length")
        if len(set(seqs)) != len(seqs):
            raise InvalidArg("a sequence appears twice in one batch")
        if any(c < 0 for c in counts):
            raise InvalidArg("negative count")
        for sid in seqs:
            self._get(sid)
        trial = copy.deepcopy(self)
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for sid, c in zip(seqs, counts):
            trial._append_one(sid, c, slots, pairs)
        self.__dict__.update(trial.__dict__)
        return np.asarray(slots, dtype=np.int64), np.asarray(pairs, dtype=np.int32).reshape(-1, 2)

    # -- views ---------------------------------------------------------------------
    def length(self, sid: int) -> int:
        return self._get(sid).length

    def table(self, sid: int) -> List[int]:
        return list(self._get(sid).table)

    def block_tables(self, seqs: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
        """Dense int32 tables ``[n][max_blocks]`` padded with -1, and the context lengths."""
        out = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, sid in enumerate(seqs):
            s = self._get(int(sid))
            if len(s.table) > max_blocks:
                raise InvalidArg("table longer than max_blocks")
            out[i, :len(s.table)] = s.table
            lens[i] = s.length
        return out, lens

    def stats(self) -> Dict[str, int]:
        used = sum(1 for r in self.refcount if r > 0)
        logical_blocks = sum(len(s.table) for s in self.seqs.values())
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "used_blocks": used,
            "sum_refcount": sum(self.refcount),
            "num_seqs": len(self.seqs),
            "logical_tokens": sum(s.length for s in self.seqs.values()),
            "logical_blocks": logical_blocks,
            "allocated_slots": used * self.block_size,
            "table_bytes": 4 * logical_blocks,
        }

    def free_list(self) -> List[int]:
        return list(self.free)
