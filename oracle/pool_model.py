"""Block pool model: free list, refcounts and per-sequence block tables.

Sources
-------
* "PagedAttention Internals", sections "Fixed-Size KV Blocks" (the cache is cut
  into fixed-size blocks; a sequence gets another block only when its current
  one is full; any free block will do), "The Block Table Map" (a per-sequence
  table from logical block to physical block, growing by one entry per new
  block) and "Sharing And Dynamic Growth" (requests hold only the blocks they
  need and release them when they finish).
* "pagedattention" topic page, third paragraph (blocks handed out one at a
  time as tokens arrive) and fourth paragraph plus the comparison table's
  "Sharing" row (a common prefix points at the same physical blocks and is
  copied on write only where the sharers diverge).
* "inference-acceleration-pagedattention-vllm" chapter: pages are allocated
  only as a sequence grows, one whole page at a time.

The pages leave the placement policy open ("any suitable free block").  To make
allocator state comparable bit for bit, one policy is fixed here and in the
GPU library's host pool, each written independently:

1. The free list is a double-ended queue seeded with the caller's order.
   Allocation takes the head; released blocks go to the tail, in the logical
   order of the releasing sequence's table.
2. Allocation is lazy: a token written at position ``len`` with
   ``len % P == 0`` takes a new block (the previous one, if any, is full).
3. Copy-on-write: a token written into a partly filled last block whose
   refcount is above one takes a fresh block first.  The pair (old, new) is
   reported so the caller can copy the block's contents; the old block's
   refcount drops by one.  Sharers are served in the order of the call's
   sequence list, so the last remaining sharer writes in place.
4. ``fork`` copies the parent's table and length and adds one reference to
   every block.
5. A call that needs more blocks than are free fails and changes nothing.
6. Slot of logical token t: ``table[t // P] * P + t % P``.
"""
from __future__ import annotations

import copy
from collections import deque
from typing import Dict, Iterable, List, Optional, Sequence, Tuple


class PoolError(Exception):
    """Base of the pool's failures."""


class NoBlocks(PoolError):
    """The free list cannot cover the request."""


class BadSeq(PoolError):
    """Unknown or already released sequence id."""


class InvalidArg(PoolError):
    """Malformed request."""


class PoolModel:
    """Slow, obviously-correct model of the block pool."""

    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks < 0 or block_size <= 0:
            raise InvalidArg("bad pool shape")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: deque = deque(order)
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}
        self.next_id = 0

    # -- sequences ---------------------------------------------------------
    def seq_create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lengths[sid] = 0
        return sid

    def _live(self, sid: int):
        if sid not in self.tables:
            raise BadSeq(f"sequence {sid} is not live")

    def append_slots(self, seqs: Sequence[int], n_new: Sequence[int]
                     ) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Append ``n_new[i]`` tokens to ``seqs[i]``, in call order.

        Returns the slot of every new token (in call order) and the
        copy-on-write pairs (source block, destination block) in the order
        they were taken.  All-or-nothing.
        """
        seqs = [int(s) for s in seqs]
        n_new = [int(n) for n in n_new]
        if len(seqs) != len(n_new):
            raise InvalidArg("seqs and n_new differ in length")
        for s in seqs:
            self._live(s)
        if len(set(seqs)) != len(seqs):
            raise InvalidArg("a sequence appears twice in one call")
        if any(n < 0 for n in n_new):
            raise InvalidArg("negative token count")
        saved = (copy.copy(self.free), list(self.ref),
                 {k: list(v) for k, v in self.tables.items()}, dict(self.lengths))
        try:
            return self._append(seqs, n_new)
        except PoolError:
            self.free, self.ref, self.tables, self.lengths = saved
            raise

    def _take(self) -> int:
        if not self.free:
            raise NoBlocks("free list exhausted")
        blk = self.free.popleft()
        assert self.ref[blk] == 0
        self.ref[blk] = 1
        return blk

    def _append(self, seqs, n_new):
        p = self.block_size
        slots: List[int] = []
        cow: List[Tuple[int, int]] = []
        for sid, n in zip(seqs, n_new):
            tab = self.tables[sid]
            for _ in range(n):
                pos = self.lengths[sid]
                if pos % p == 0:
                    assert len(tab) == pos // p
                    tab.append(self._take())
                elif self.ref[tab[-1]] > 1:
                    src = tab[-1]
                    dst = self._take()
                    self.ref[src] -= 1
                    cow.append((src, dst))
                    tab[-1] = dst
                slots.append(tab[pos // p] * p + pos % p)
                self.lengths[sid] = pos + 1
        return slots, cow

    def fork(self, parent: int) -> int:
        self._live(parent)
        child = self.seq_create()
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for blk in self.tables[child]:
            self.ref[blk] += 1
        return child

    def free_seq(self, sid: int) -> None:
        self._live(sid)
        for blk in self.tables.pop(sid):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.append(blk)
        del self.lengths[sid]

    def set_table(self, sid: int, phys: Sequence[int], length: int) -> None:
        """Place an empty sequence on the given free blocks, in logical order."""
        self._live(sid)
        phys = [int(x) for x in phys]
        if self.tables[sid] or self.lengths[sid]:
            raise InvalidArg("set_table needs an empty sequence")
        if length < 0 or -(-length // self.block_size) != len(phys):
            raise InvalidArg("length does not match the number of blocks")
        if len(set(phys)) != len(phys):
            raise InvalidArg("repeated block")
        for blk in phys:
            if not (0 <= blk < self.num_blocks) or self.ref[blk] != 0:
                raise InvalidArg(f"block {blk} is not free")
        taken = set(phys)
        self.free = deque(b for b in self.free if b not in taken)
        for blk in phys:
            self.ref[blk] = 1
        self.tables[sid] = phys
        self.lengths[sid] = int(length)

    # -- queries -----------------------------------------------------------
    def slot(self, sid: int, t: int) -> int:
        self._live(sid)
        if not 0 <= t < self.lengths[sid]:
            raise InvalidArg("token outside the sequence")
        p = self.block_size
        return self.tables[sid][t // p] * p + t % p

    def slots_of(self, sid: int) -> List[int]:
        return [self.slot(sid, t) for t in range(self.lengths[sid])]

    def stats(self) -> Dict[str, float]:
        """Pool occupancy; a shared block and its tokens are counted once."""
        p = self.block_size
        fill = [0] * self.num_blocks
        for sid, tab in self.tables.items():
            n = self.lengths[sid]
            for j, blk in enumerate(tab):
                fill[blk] = max(fill[blk], min(p, n - j * p))
        used = [b for b in range(self.num_blocks) if self.ref[b] > 0]
        alloc = len(used) * p
        live = sum(fill[b] for b in used)
        return {"num_blocks": self.num_blocks, "free_blocks": len(self.free),
                "used_blocks": len(used), "allocated_slots": alloc,
                "live_tokens": live, "wasted_slots": alloc - live,
                "fragmentation": (alloc - live) / alloc if alloc else 0.0,
                "num_seqs": len(self.tables)}

    def export(self) -> Tuple[List[int], List[int]]:
        """(free list in order, refcount of every block)."""
        return list(self.free), list(self.ref)

    def check_invariants(self) -> None:
        """Bookkeeping identities that hold after every operation."""
        p = self.block_size
        counted = [0] * self.num_blocks
        for sid, tab in self.tables.items():
            assert len(tab) == -(-self.lengths[sid] // p)
            for blk in tab:
                counted[blk] += 1
        assert counted == self.ref
        free = list(self.free)
        assert len(set(free)) == len(free)
        assert all(self.ref[b] == 0 for b in free)
        assert len(free) + sum(1 for r in self.ref if r > 0) == self.num_blocks
