"""Oracle: block bookkeeping twin (LIFO free list + refcounts) — test infrastructure only.

Follows "P3: native paged-KV continuous-batching sampler", section "Design > paged.py":
  * BlockAllocator: LIFO free list plus refcounts; freeing a block whose refcount is already 0
    is an error (a double free would put one block on the list twice and give it to two
    sequences); check_consistent proves free + referenced == total with no duplicates.
  * Growth is all-or-nothing (ensure_capacity); running out is a typed error, never a silent
    truncation ("Optional paged KV cache (vLLM-style) — v1 design", section "Design":
    alloc pops the free list or throws PagedPoolExhausted).
  * A block with refcount > 1 is read-only for everyone, owner included: slots() refuses a
    write into it. Sharing adopts a running sequence's leading FULL blocks (P3 page,
    "Design > engine.py", Prefix sharing).

Readings where the page leaves a step open (each listed in the design notes):
  * A fresh pool hands out ids 0, 1, 2, ... (stack initialised as [NB-1, ..., 1, 0], top last).
  * Multi-id calls apply ids in array order, and are all-or-nothing: on any error no state
    changes.
  * incref of a block with refcount 0 is an error (sharing needs a live owner).
  * A slot is block * block_size + offset.
"""
from __future__ import annotations

from collections import Counter
from typing import List, Sequence


class AllocatorError(Exception):
    pass


class PoolExhausted(AllocatorError):
    pass


class DoubleFree(AllocatorError):
    pass


class SharedWrite(AllocatorError):
    pass


class InvalidBlock(AllocatorError):
    pass


def slot_of(block: int, pos: int, block_size: int) -> int:
    """Flat slot of position pos inside its block: block * block_size + pos % block_size."""
    return block * block_size + pos % block_size


class BlockAllocator:
    def __init__(self, num_blocks: int):
        if num_blocks < 0:
            raise InvalidBlock("num_blocks must be >= 0")
        self.num_blocks = int(num_blocks)
        self.free_stack: List[int] = list(range(self.num_blocks - 1, -1, -1))  # top = last
        self.refcount: List[int] = [0] * self.num_blocks

    # ---- queries ---------------------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free_stack)

    def _check_id(self, i: int) -> None:
        if not 0 <= i < self.num_blocks:
            raise InvalidBlock(f"block id {i} outside [0, {self.num_blocks})")

    # ---- events ----------------------------------------------------------------------------
    def allocate(self, n: int) -> List[int]:
        """Pop n ids off the free stack (in pop order), each with refcount 1; all or nothing."""
        if n < 0:
            raise InvalidBlock("negative count")
        if n > len(self.free_stack):
            raise PoolExhausted(f"need {n} blocks, {len(self.free_stack)} free")
        ids = [self.free_stack.pop() for _ in range(n)]
        for i in ids:
            self.refcount[i] = 1
        return ids

    def incref(self, ids: Sequence[int]) -> None:
        """Share: add one reference to each id; every id must be live."""
        ids = [int(i) for i in ids]
        for i in ids:
            self._check_id(i)
            if self.refcount[i] < 1:
                raise InvalidBlock(f"incref of free block {i}")
        for i in ids:
            self.refcount[i] += 1

    def free(self, ids: Sequence[int]) -> None:
        """Drop one reference per id, in array order; a block reaching 0 goes on the stack."""
        ids = [int(i) for i in ids]
        for i in ids:
            self._check_id(i)
        for i, c in Counter(ids).items():
            if self.refcount[i] < c:
                raise DoubleFree(f"free of block {i} with refcount {self.refcount[i]}")
        for i in ids:
            self.refcount[i] -= 1
            if self.refcount[i] == 0:
                self.free_stack.append(i)

    def check_consistent(self) -> bool:
        """free + referenced == total, no duplicate on the stack, no stack member referenced."""
        if len(set(self.free_stack)) != len(self.free_stack):
            return False
        if any(self.refcount[i] != 0 for i in self.free_stack):
            return False
        if any(r < 0 for r in self.refcount):
            return False
        referenced = sum(1 for r in self.refcount if r > 0)
        return len(self.free_stack) + referenced == self.num_blocks

    def slots(self, block_table_row: Sequence[int], start_pos: int, n_new: int,
              block_size: int) -> List[int]:
        """Slots of positions start_pos .. start_pos + n_new - 1 of one sequence.

        Refuses a position whose block is shared (refcount > 1) or not live.
        """
        if block_size <= 0 or start_pos < 0 or n_new < 0:
            raise InvalidBlock("bad slot-mapping arguments")
        row = [int(x) for x in block_table_row]
        out = []
        for p in range(start_pos, start_pos + n_new):
            j = p // block_size
            if j >= len(row):
                raise InvalidBlock(f"position {p} past the block table")
            blk = row[j]
            self._check_id(blk)
            if self.refcount[blk] == 0:
                raise InvalidBlock(f"block {blk} is free")
            if self.refcount[blk] > 1:
                raise SharedWrite(f"block {blk} is shared (refcount {self.refcount[blk]})")
            out.append(slot_of(blk, p, block_size))
        return out
