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
  * Preemption by swapping: the blocks of sequences that must wait are moved
    to host memory and brought back when device blocks are free again
    ([P2] section 4 "scheduling: first come first served plus preemption";
    [P4] "Preemption", swapping).
  * Automatic prefix caching: a full block is found again by a key hashed
    from its own tokens and every token before it, and two blocks are the
    same only if that whole run of tokens is the same ([P4] the note on
    identical KV blocks, and the prefix-caching paragraph; [P2] section 3).

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
  * Swapping works on whole sharing groups: every holder of a block moves with
    it (beams of one request move together), so a listed set whose blocks are
    also held by an unlisted sequence is refused.  The host tier has its own
    FIFO queue of host block ids 0, 1, 2, ...  Swap-out meets the listed
    sequences' blocks in list order, then logical order; each distinct device
    block takes the next host block, which inherits its refcount, and the
    device block joins the device queue's tail.  Swap-in mirrors it.  Both are
    all or nothing.  A swapped-out sequence can only be swapped in or freed.
  * Prefix keys.  key(block 0) = FNV-1a-64 of the 8 little-endian bytes of 0
    then the block's B token ids as 4-byte little-endian integers; key(block
    i) chains the same way from key(block i-1).  A block is registered when an
    append that carries token ids fills it and its key is not yet registered.
    A lookup hits only if the key is registered and the block's stored
    parent key and tokens equal the query (so a hash collision is a miss).
    A new sequence takes the longest run of leading hits, at most
    (n - 1) // B blocks of its n prompt tokens (one token is always left to
    compute).  A hit block with refcount 0 leaves the free queue wherever it
    sits.  Freed blocks keep their key while they wait in the queue; a block
    loses it when it is popped for new use (eviction, oldest freed first) or
    moved to the host tier.  An append without token ids stops a sequence's
    key chain; blocks brought back from the host are not registered again.
  * Rollback (speculative decoding stages KV positions and drops the ones its
    verification rejects, [P3] section 5).  truncate(s, n') keeps the first n'
    tokens: the table keeps ceil(n' / B) blocks and the rest are released in
    logical order, as a free does.  A truncated sequence stops being keyed (the
    ids of the tokens it keeps are not all held).  A block that becomes
    partly filled keeps its bytes and any key until it is written again: an
    append that writes in place into a keyed last block first drops its key,
    and a shared one is copied on write as usual.

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


class WrongTier(PoolError):
    """The sequence is on the other tier (swapped out, or not swapped out)."""


FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit (Fowler, Noll, Vo): xor each byte in, then multiply by the prime, modulo 2^64."""
    h = FNV64_OFFSET
    for byte in data:
        h = ((h ^ byte) * FNV64_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def block_key(parent: int, tokens: Sequence[int]) -> int:
    """Prefix key of a full block whose preceding block has key ``parent`` (0 for the first block)."""
    data = int(parent).to_bytes(8, "little") + b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return fnv1a64(data)


@dataclass
class _Seq:
    table: List[int] = field(default_factory=list)
    length: int = 0
    on_host: bool = False  # swapped out: the table holds host block ids
    tracked: bool = True  # every token so far came with its id: the key chain is known
    last_key: int = 0  # key of the last full block (0 before the first)
    partial: List[int] = field(default_factory=list)  # token ids of the partly filled last block


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None,
                 host_blocks: int = 0):
        if num_blocks <= 0 or block_size <= 0 or host_blocks < 0:
            raise InvalidArg("num_blocks and block_size must be positive, host_blocks not negative")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: deque = deque(order)
        self.refcount = [0] * num_blocks
        self.seqs: Dict[int, _Seq] = {}
        self.next_id = 0
        self.host_blocks = host_blocks
        self.host_free: deque = deque(range(host_blocks))
        self.host_refcount = [0] * host_blocks
        self.cached: Dict[int, int] = {}  # prefix key -> device block
        self.block_keys: Dict[int, Tuple[int, int, Tuple[int, ...]]] = {}  # block -> (key, parent key, tokens)

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

    def _on_device(self, sid: int) -> _Seq:
        s = self._get(sid)
        if s.on_host:
            raise WrongTier(sid)
        return s

    def fork(self, parent: int) -> int:
        """New sequence sharing every block of ``parent``; each shared block's count rises by one."""
        p = self._on_device(parent)
        sid = self.create()
        self.seqs[sid] = _Seq(table=list(p.table), length=p.length, tracked=p.tracked, last_key=p.last_key,
                              partial=list(p.partial))
        for b in p.table:
            self.refcount[b] += 1
        return sid

    def free_seq(self, sid: int) -> None:
        """Release ``sid``: counts drop in logical order; blocks reaching zero join the queue's tail."""
        s = self._get(sid)
        refcount, queue = (self.host_refcount, self.host_free) if s.on_host else (self.refcount, self.free)
        for b in s.table:
            refcount[b] -= 1
            if refcount[b] == 0:
                queue.append(b)
        del self.seqs[sid]

    # -- appends ---------------------------------------------------------------
    def _pop(self) -> int:
        if not self.free:
            raise OutOfBlocks()
        b = self.free.popleft()
        self._forget(b)  # a cached block taken for new use loses its key
        self.refcount[b] = 1
        return b

    def _forget(self, b: int) -> None:
        if b in self.block_keys:
            key = self.block_keys.pop(b)[0]
            if self.cached.get(key) == b:
                del self.cached[key]

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
            else:
                self._forget(last)  # written in place: a key it kept from before a rollback no longer holds
        for p in range(s.length, s.length + count):
            if p % B == 0:
                s.table.append(self._pop())
            slots.append(s.table[p // B] * B + p % B)
        s.length += count

    def _track(self, sid: int, ids: Sequence[int]) -> None:
        """Extend sid's key chain by the ids just appended, registering every block they fill."""
        s = self.seqs[sid]
        B = self.block_size
        if not s.tracked:
            return
        pos = s.length - len(ids)
        for t in ids:
            s.partial.append(int(t))
            if len(s.partial) == B:
                b = s.table[pos // B]
                key = block_key(s.last_key, s.partial)
                if key not in self.cached:
                    self.cached[key] = b
                    self.block_keys[b] = (key, s.last_key, tuple(s.partial))
                s.last_key = key
                s.partial = []
            pos += 1

    def append(self, seqs: Sequence[int], counts: Sequence[int],
               token_ids: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Append ``counts[i]`` tokens to ``seqs[i]``, in order; all or nothing.

        Returns ``(slots int64[sum counts], pairs int32[k][2])``; slots are in
        sequence-major, position order.  Raises OutOfBlocks (state unchanged)
        when the pool cannot hold the whole batch.  ``token_ids`` (sequence-
        major, one per new token) extends the sequences' prefix keys; without
        it, the appended sequences stop being keyed.
        """
        seqs = [int(x) for x in seqs]
        counts = [int(c) for c in counts]
        if len(seqs) != len(counts):
            raise InvalidArg("seqs and counts differ in length")
        if token_ids is not None and len(token_ids) != sum(max(c, 0) for c in counts):
            raise InvalidArg("one token id per appended token")
        if len(set(seqs)) != len(seqs):
            raise InvalidArg("a sequence appears twice in one batch")
        if any(c < 0 for c in counts):
            raise InvalidArg("negative count")
        for sid in seqs:
            self._get(sid)
        for sid in seqs:
            self._on_device(sid)
        trial = copy.deepcopy(self)
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for sid, c in zip(seqs, counts):
            trial._append_one(sid, c, slots, pairs)
        k = 0
        for sid, c in zip(seqs, counts):
            if c == 0:
                continue
            if token_ids is None:
                trial.seqs[sid].tracked = False
                trial.seqs[sid].partial = []
            else:
                trial._track(sid, token_ids[k:k + c])
            k += c
        self.__dict__.update(trial.__dict__)
        return np.asarray(slots, dtype=np.int64), np.asarray(pairs, dtype=np.int32).reshape(-1, 2)

    def truncate(self, sid: int, new_len: int) -> None:
        """Keep the first ``new_len`` tokens of ``sid``; blocks past ceil(new_len / B) are released in logical order."""
        s = self._on_device(sid)
        new_len = int(new_len)
        if new_len < 0 or new_len > s.length:
            raise InvalidArg("new length outside [0, length]")
        if new_len == s.length:
            return
        keep = -(-new_len // self.block_size)
        for b in s.table[keep:]:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        s.table = s.table[:keep]
        s.length = new_len
        s.tracked = False
        s.partial = []

    # -- prefix caching ----------------------------------------------------------------
    def create_prefixed(self, token_ids: Sequence[int]) -> Tuple[int, int]:
        """New sequence whose prompt is ``token_ids``: it starts with the longest run of cached leading blocks.

        Returns ``(sequence id, cached tokens)``; the caller appends the
        remaining ``token_ids[cached:]`` (with their ids) and computes only
        their keys and values.
        """
        ids = [int(t) for t in token_ids]
        B = self.block_size
        sid = self.create()
        s = self.seqs[sid]
        for i in range((len(ids) - 1) // B if ids else 0):
            toks = tuple(ids[i * B:(i + 1) * B])
            key = block_key(s.last_key, toks)
            b = self.cached.get(key)
            if b is None or self.block_keys[b] != (key, s.last_key, toks):
                break
            if self.refcount[b] == 0:
                self.free.remove(b)
            self.refcount[b] += 1
            s.table.append(b)
            s.length += B
            s.last_key = key
        return sid, s.length

    # -- swapping --------------------------------------------------------------------
    def _swap(self, seqs: Sequence[int], out: bool) -> np.ndarray:
        seqs = [int(x) for x in seqs]
        if len(set(seqs)) != len(seqs):
            raise InvalidArg("a sequence appears twice in one swap")
        for sid in seqs:
            self._get(sid)
        for sid in seqs:
            if self.seqs[sid].on_host == out:
                raise WrongTier(sid)
        src_ref, src_queue = (self.refcount, self.free) if out else (self.host_refcount, self.host_free)
        dst_ref, dst_queue = (self.host_refcount, self.host_free) if out else (self.refcount, self.free)
        # the blocks in the order they are met, and how often the listed tables hold each
        met: List[int] = []
        held: Dict[int, int] = {}
        for sid in seqs:
            for b in self.seqs[sid].table:
                if b not in held:
                    held[b] = 0
                    met.append(b)
                held[b] += 1
        if any(held[b] != src_ref[b] for b in met):
            raise InvalidArg("a block of the listed sequences is also held by an unlisted one")
        if len(met) > len(dst_queue):
            raise OutOfBlocks()
        moved: Dict[int, int] = {}
        for b in met:
            if out:
                self._forget(b)  # keys name device blocks only
            nb = dst_queue.popleft()
            if not out:
                self._forget(nb)
            dst_ref[nb] = src_ref[b]
            src_ref[b] = 0
            src_queue.append(b)
            moved[b] = nb
        for sid in seqs:
            s = self.seqs[sid]
            s.table = [moved[b] for b in s.table]
            s.on_host = out
        return np.asarray([(b, moved[b]) for b in met], dtype=np.int32).reshape(-1, 2)

    def swap_out(self, seqs: Sequence[int]) -> np.ndarray:
        """Move the listed sequences (a whole sharing group) to the host tier.

        Returns int32 pairs (device block, host block) in the order the blocks
        are met; the caller copies each device block to its host block before
        the freed device blocks are written again.  Raises InvalidArg (a block
        also held outside the list), WrongTier (already on the host),
        OutOfBlocks (host tier too small); the state is then unchanged.
        """
        return self._swap(seqs, True)

    def swap_in(self, seqs: Sequence[int]) -> np.ndarray:
        """Bring swapped-out sequences back; pairs are (host block, device block)."""
        return self._swap(seqs, False)

    def on_host(self, sid: int) -> bool:
        return self._get(sid).on_host

    def host_free_list(self) -> List[int]:
        return list(self.host_free)

    # -- views ---------------------------------------------------------------------
    def length(self, sid: int) -> int:
        return self._get(sid).length

    def table(self, sid: int) -> List[int]:
        return list(self._get(sid).table)

    def block_tables(self, seqs: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
        """Dense int32 tables ``[n][max_blocks]`` padded with -1, and the context lengths."""
        out = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for sid in seqs:
            self._on_device(int(sid))
        for i, sid in enumerate(seqs):
            s = self._get(int(sid))
            if len(s.table) > max_blocks:
                raise InvalidArg("table longer than max_blocks")
            out[i, :len(s.table)] = s.table
            lens[i] = s.length
        return out, lens

    def stats(self) -> Dict[str, int]:
        used = sum(1 for r in self.refcount if r > 0)
        resident = [s for s in self.seqs.values() if not s.on_host]
        swapped = [s for s in self.seqs.values() if s.on_host]
        logical_blocks = sum(len(s.table) for s in resident)
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "used_blocks": used,
            "sum_refcount": sum(self.refcount),
            "num_seqs": len(self.seqs),
            "logical_tokens": sum(s.length for s in resident),
            "logical_blocks": logical_blocks,
            "allocated_slots": used * self.block_size,
            "table_bytes": 4 * logical_blocks,
            "host_blocks": self.host_blocks,
            "host_free_blocks": len(self.host_free),
            "host_used_blocks": sum(1 for r in self.host_refcount if r > 0),
            "swapped_seqs": len(swapped),
            "swapped_tokens": sum(s.length for s in swapped),
            "cached_blocks": len(self.cached),
            "cached_free_blocks": sum(1 for b in self.free if b in self.block_keys),
        }

    def free_list(self) -> List[int]:
        return list(self.free)
