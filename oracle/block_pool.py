"""Plain Python KV block pool and step-input builder (test infrastructure only).

What the pages fix (llm-stack-book 7.3 "vLLM: Architecture, PagedAttention &
Internals", sections "The free list and the block table", "Copy-on-write for
shared blocks" and "The forward step in detail"; modernaiengineering.com lesson
13.15 "vLLM: High-Throughput Serving with PagedAttention", sections "How
PagedAttention stores a request" and "How PagedAttention shares memory"):

* the pool is a free list of physical block ids; a block is taken from the end
  of the list and a released block goes back onto the end;
* a sequence of n tokens holds ceil(n / block_size) blocks, taken one at a time
  as decode crosses block boundaries, never ahead of need;
* every held block carries a reference count; sharing a block (parallel
  sampling, beam search, prefix reuse) raises it, releasing lowers it, and a
  block returns to the free list only when its count reaches zero;
* a sequence about to write into a block others still hold first gets a
  private copy: a fresh block, the old block's count lowered, its table entry
  repointed, and a (source, destination) copy to run on the GPU;
* each step, token position p of a sequence writes its K/V to slot
  table[p // block_size] * block_size + p % block_size, and the sequence's
  whole block table is handed to attention.

Where the pages leave a choice open this module takes the plain reading:
growing a table means covering one more position (a table already long enough
takes nothing); taking more blocks than are free is an error that changes
nothing; releasing walks the table in order.
"""
from __future__ import annotations

import math


class PoolError(RuntimeError):
    """Raised for operations the pool cannot perform (no free blocks, bad ids)."""


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks < 0 or block_size <= 0:
            raise PoolError("bad pool shape")
        self.block_size = block_size
        # The free list; its last entry is handed out first.
        self.free = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(self.free) != list(range(num_blocks)):
            raise PoolError("free_order must be a permutation of the block ids")
        self.refs: dict[int, int] = {}

    # ---------------------------------------------------------------- queries
    def blocks_for(self, num_tokens: int) -> int:
        return math.ceil(num_tokens / self.block_size) if num_tokens > 0 else 0

    def num_free(self) -> int:
        return len(self.free)

    def ref_count(self, block: int) -> int:
        return self.refs.get(block, 0)

    def can_allocate(self, num_tokens: int) -> bool:
        return self.blocks_for(num_tokens) <= len(self.free)

    # ------------------------------------------------------------- mutation
    def _take(self) -> int:
        if not self.free:
            raise PoolError("no free block")
        b = self.free.pop()
        self.refs[b] = 1
        return b

    def allocate(self, num_tokens: int) -> list[int]:
        """A fresh block table for ``num_tokens`` tokens (all or nothing)."""
        n = self.blocks_for(num_tokens)
        if n > len(self.free):
            raise PoolError("not enough free blocks")
        return [self._take() for _ in range(n)]

    def append_slot(self, table: list[int], cur_len: int):
        """Make ``table`` cover token position ``cur_len`` (the token about to
        be written). Returns the block taken, or None when the table already
        covers that position, which is every step except the ones that start a
        new block."""
        need = cur_len // self.block_size + 1
        if len(table) >= need:
            return None
        if need - len(table) > len(self.free):
            raise PoolError("not enough free blocks")
        taken = None
        while len(table) < need:
            taken = self._take()
            table.append(taken)
        return taken

    def share(self, blocks) -> None:
        """One more holder for each block (each must be held already)."""
        for b in blocks:
            if self.refs.get(b, 0) <= 0:
                raise PoolError(f"block {b} is not held")
        for b in blocks:
            self.refs[b] += 1

    def release(self, blocks) -> None:
        """One holder fewer for each block, in order; a block nobody holds goes
        back onto the free list."""
        for b in blocks:
            if self.refs.get(b, 0) <= 0:
                raise PoolError(f"block {b} is not held")
        for b in blocks:
            self.refs[b] -= 1
            if self.refs[b] == 0:
                del self.refs[b]
                self.free.append(b)

    def make_writable(self, table: list[int], idx: int):
        """Copy-on-write for ``table[idx]``: if others hold the block too, the
        table gets a fresh private block and the copy (source, destination) is
        returned; otherwise None."""
        b = table[idx]
        if self.refs.get(b, 0) <= 0:
            raise PoolError(f"block {b} is not held")
        if self.refs[b] == 1:
            return None
        if not self.free:
            raise PoolError("no free block")
        fresh = self._take()
        self.refs[b] -= 1
        table[idx] = fresh
        return (b, fresh)


def prepare_step(tables, num_computed, num_new, block_size: int, max_blocks: int):
    """Inputs of one engine step for sequences that each process ``num_new[i]``
    tokens (a prompt chunk or one decode token) after ``num_computed[i]``
    stored ones.

    Returns (slot_mapping, positions, block_tables, context_lens): for every
    token, in sequence order, its slot and position; every table padded with
    -1 to ``max_blocks`` entries; and each sequence's length after the step.
    """
    slots, positions, rows, lens = [], [], [], []
    for table, done, new in zip(tables, num_computed, num_new):
        if len(table) > max_blocks:
            raise PoolError("block table longer than max_blocks")
        for p in range(done, done + new):
            blk = p // block_size
            if blk >= len(table):
                raise PoolError("block table does not cover the step's tokens")
            slots.append(table[blk] * block_size + p % block_size)
            positions.append(p)
        rows.append(list(table) + [-1] * (max_blocks - len(table)))
        lens.append(done + new)
    return slots, positions, rows, lens
