"""Host-side block allocator used to build paged-KV inputs.

Bookkeeping only (block ids, reference counts, per-sequence block tables);
it moves no K/V data itself. It follows the paging scheme of the pages:

* KV cache split into fixed-size blocks of ``block_size`` tokens that may sit
  anywhere in a pool; each sequence keeps a block table mapping its logical
  blocks to physical ones ("PagedAttention 是如何工作的" / "分页式KV缓存"
  sections of the devpress.csdn.net page; section 2.2 of the betteryeah.com
  page).
* blocks are handed out on demand as a sequence grows and returned when it
  finishes (step 7 "内存回收" of the workflow list on the devpress page;
  section 2.2 of the betteryeah page).
* parallel sampling shares the prompt's blocks through the block tables, with a
  reference count per physical block and copy-on-write before a sharer writes
  into a shared block (the parallel-sampling answer in the FAQ of the
  aidocs.cortexgrid.cn page).

Copy-on-write events are recorded as ``(src_block, dst_block)`` pairs; the
caller replays them on its pool in order.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


class AllocatorError(RuntimeError):
    pass


@dataclass
class Sequence:
    table: list = field(default_factory=list)  # physical block ids, logical order
    length: int = 0                             # tokens stored


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int, rng: np.random.Generator | None = None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocatorError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = np.arange(num_blocks) if rng is None else rng.permutation(num_blocks)
        # pop() takes from the end: reverse so the first handed out is order[0]
        self.free_list = [int(b) for b in order[::-1]]
        self.refcount = np.zeros(num_blocks, dtype=np.int64)
        self.copies: list[tuple[int, int]] = []  # copy-on-write log

    # -- block level -------------------------------------------------------
    def alloc(self) -> int:
        if not self.free_list:
            raise AllocatorError("out of KV blocks")
        b = self.free_list.pop()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def release(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise AllocatorError(f"double free of block {b}")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free_list.append(int(b))

    @property
    def num_free(self) -> int:
        return len(self.free_list)

    # -- sequence level ----------------------------------------------------
    def new_sequence(self) -> Sequence:
        return Sequence()

    def append(self, seq: Sequence, n: int) -> list[int]:
        """Reserve slots for ``n`` new tokens at the end of ``seq``.

        Returns the slot index ``block * block_size + offset`` of each new
        token. A new block is taken only when the last one is full; a shared
        last block is copied first (copy-on-write)."""
        slots = []
        bs = self.block_size
        for _ in range(int(n)):
            off = seq.length % bs
            if off == 0:
                seq.table.append(self.alloc())
            else:
                last = seq.table[-1]
                if self.refcount[last] > 1:
                    fresh = self.alloc()
                    self.copies.append((int(last), int(fresh)))
                    self.release(last)
                    seq.table[-1] = fresh
            slots.append(seq.table[-1] * bs + off)
            seq.length += 1
        return slots

    def fork(self, seq: Sequence) -> Sequence:
        """New sequence sharing every block of ``seq`` (refcount + 1 each)."""
        for b in seq.table:
            self.refcount[b] += 1
        return Sequence(table=list(seq.table), length=seq.length)

    def free(self, seq: Sequence) -> None:
        for b in seq.table:
            self.release(b)
        seq.table = []
        seq.length = 0

    def table_refs(self, seqs) -> int:
        return sum(len(s.table) for s in seqs)
