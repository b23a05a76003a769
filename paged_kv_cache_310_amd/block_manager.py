"""Host-side KV block manager: on-demand allocation, reference counts,
fork and copy-on-write, and the fragmentation arithmetic.

It runs on the CPU and never touches device memory.  It decides *where* a
token goes (the slot mapping), which blocks a sequence owns (its block
table) and which blocks must be duplicated before a write (the copy list).
The device operations that act on those decisions live in the HIP library.

Sources: the "Efficient Memory Management for Large Language Model Serving
with PagedAttention" pages --
* zeroshotmind.com essay, "Paging the cache": fixed-size blocks (16 tokens by
  default), allocated one at a time as a sequence grows; a sequence holds
  exactly the blocks its length needs, at most one of them partly filled.
* same essay, "Block tables: logical order, physical scatter": one table per
  sequence maps logical block index -> physical block number.
* same essay, "Sharing a prefix without copying it": shared blocks carry a
  reference count; a write into a shared block duplicates that one block,
  repoints the writer at the copy and decrements the original's count.
* same essay, "The fragmentation arithmetic" and "The memory you allocate
  but never use": tail slack is at most ``block_size - 1`` tokens; the
  contiguous scheme wastes ``cap - used`` tokens per request.
"""

from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np


class PoolExhausted(RuntimeError):
    """Raised when a block is needed and the free list is empty."""


def blocks_needed(length: int, block_size: int) -> int:
    """Blocks a sequence of ``length`` tokens holds: ``ceil(length / bs)``."""
    return -(-int(length) // int(block_size))


def tail_slack(length: int, block_size: int) -> int:
    """Unused slots in the sequence's last block (0 when it is full)."""
    return blocks_needed(length, block_size) * block_size - int(length)


def paged_waste_fraction(lengths: Iterable[int], block_size: int) -> float:
    """Fraction of allocated KV slots that hold no token, paged scheme."""
    lengths = [int(x) for x in lengths]
    allocated = sum(blocks_needed(x, block_size) for x in lengths) * block_size
    if allocated == 0:
        return 0.0
    return (allocated - sum(lengths)) / allocated


def contiguous_waste_tokens(reserved: int, used: int) -> int:
    """Internal fragmentation of a contiguous max-length reservation."""
    return int(reserved) - int(used)


class BlockManager:
    """Physical block pool with per-sequence block tables.

    ``free_order`` fixes which physical block each allocation returns
    (first in, first out), so a seeded permutation scatters logical blocks
    across the pool reproducibly.
    """

    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Iterable[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self.free: deque = deque(order)
        self.refcount = np.zeros(num_blocks, dtype=np.int64)
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}

    # -- blocks ---------------------------------------------------------
    def allocate(self) -> int:
        if not self.free:
            raise PoolExhausted(f"all {self.num_blocks} blocks are in use")
        block = self.free.popleft()
        self.refcount[block] = 1
        return block

    def _release(self, block: int) -> None:
        self.refcount[block] -= 1
        if self.refcount[block] < 0:
            raise AssertionError(f"refcount of block {block} went negative")
        if self.refcount[block] == 0:
            self.free.append(block)

    # -- sequences ------------------------------------------------------
    def add_sequence(self, seq: int, length: int = 0) -> None:
        """Register a sequence already holding ``length`` tokens."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        need = blocks_needed(length, self.block_size)
        if need > len(self.free):          # all or nothing: no partial allocation
            raise PoolExhausted(f"{need} blocks needed, {len(self.free)} free")
        self.tables[seq] = [self.allocate() for _ in range(need)]
        self.lengths[seq] = int(length)

    def append_slot(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot for the sequence's next token.

        Returns ``(slot, copy)`` where ``copy`` is ``(src, dst)`` when the
        tail block was shared and had to be duplicated first, else ``None``.
        A fresh block is taken only when the tail block is full.
        """
        n = self.lengths[seq]
        table = self.tables[seq]
        copy = None
        if n % self.block_size == 0:
            table.append(self.allocate())
        else:
            tail = table[-1]
            if self.refcount[tail] > 1:
                fresh = self.allocate()
                copy = (tail, fresh)
                self.refcount[tail] -= 1
                table[-1] = fresh
        slot = table[n // self.block_size] * self.block_size + n % self.block_size
        self.lengths[seq] = n + 1
        return slot, copy

    def fork(self, parent: int, child: int) -> None:
        """Child shares every block of the parent (reference counted)."""
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        for block in self.tables[child]:
            self.refcount[block] += 1
        self.lengths[child] = self.lengths[parent]

    def free_sequence(self, seq: int) -> None:
        for block in self.tables.pop(seq):
            self._release(block)
        del self.lengths[seq]

    # -- views ----------------------------------------------------------
    def block_table_array(self, seqs: List[int], max_blocks: int, pad: int = -1) -> np.ndarray:
        out = np.full((len(seqs), max_blocks), pad, dtype=np.int32)
        for i, seq in enumerate(seqs):
            table = self.tables[seq]
            if len(table) > max_blocks:
                raise ValueError(f"sequence {seq} holds {len(table)} > {max_blocks} blocks")
            out[i, :len(table)] = table
        return out

    def slack(self, seq: int) -> int:
        return len(self.tables[seq]) * self.block_size - self.lengths[seq]

    def check_invariants(self) -> None:
        """Reference counts equal table references; free blocks are unused;
        every sequence holds exactly ``ceil(len / bs)`` blocks."""
        refs = np.zeros(self.num_blocks, dtype=np.int64)
        for seq, table in self.tables.items():
            if len(table) != blocks_needed(self.lengths[seq], self.block_size):
                raise AssertionError(f"sequence {seq}: {len(table)} blocks for length {self.lengths[seq]}")
            for block in table:
                refs[block] += 1
        if not np.array_equal(refs, self.refcount):
            raise AssertionError("reference counts disagree with the block tables")
        free = list(self.free)
        if len(set(free)) != len(free):
            raise AssertionError("a block is on the free list twice")
        if any(refs[b] for b in free):
            raise AssertionError("a referenced block is on the free list")
        if len(free) + int((refs > 0).sum()) != self.num_blocks:
            raise AssertionError("a block is neither free nor referenced")
