"""Host block allocator used to build block tables for the synthetic workloads.

This is input generation: it decides which pool block each logical block of
each sequence occupies, exactly as a serving engine's KV manager would, and
records the per-entry fill count.  It computes no attention and no slot
numbers; the oracle and the HIP path each translate positions to slots on
their own.

What it follows:

* One pool of equal blocks handed out from a free list; a freed block is reused
  at once with no compaction ("PagedAttention 完全拆解", 原理详解（一）, Figure 7
  walk-through; the vLLM blog page on continuous batching, free-block list).
* A table entry holds a pool block id and the number of filled slots; a new
  block is taken only when the sequence's last block is full ("PagedAttention
  完全拆解", 原理详解（一）, Figure 6 walk-through).
* Per-block reference counts; writing into a shared block (count > 1) first
  copies it into a fresh block, decrements the old count and redirects the
  writer's table, while a block with count 1 is written in place ("PagedAttention
  完全拆解", 内存共享 / 引用计数, Figure 8 walk-through).
* fork / append / free as the three sequence primitives ("PagedAttention 完全拆解",
  三种原语：fork、append、free).

The free list is LIFO: ``allocate`` pops the most recently pushed block.  A
caller may seed it with any order to force the pages' example block ids.
"""

from __future__ import annotations

from dataclasses import dataclass, field


class PoolExhausted(RuntimeError):
    """Raised when an allocation finds the free list empty.  Nothing is changed
    by the failing call (all-or-nothing)."""


@dataclass
class TableEntry:
    block: int
    filled: int


@dataclass
class BlockAllocator:
    num_blocks: int
    block_size: int
    free_stack: list = field(default_factory=list)
    refcount: list = field(default_factory=list)
    tables: dict = field(default_factory=dict)   # seq id -> list[TableEntry]
    copies: list = field(default_factory=list)   # pending (src, dst) block copies
    _next_seq: int = 0

    @classmethod
    def create(cls, num_blocks: int, block_size: int, pop_order=None) -> "BlockAllocator":
        """A pool with every block free.

        ``pop_order`` lists block ids in the order successive allocations
        should receive them (default 0, 1, 2, ...).  It must be a permutation
        of ``range(num_blocks)``.
        """
        order = list(range(num_blocks)) if pop_order is None else [int(b) for b in pop_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("pop_order must be a permutation of the pool's block ids")
        a = cls(num_blocks=num_blocks, block_size=block_size)
        a.free_stack = list(reversed(order))  # top of the stack is the end of the list
        a.refcount = [0] * num_blocks
        return a

    # -- blocks ---------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free_stack)

    def allocate(self) -> int:
        if not self.free_stack:
            raise PoolExhausted("no free block")
        b = self.free_stack.pop()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def release(self, b: int) -> None:
        """Drop one reference; the block returns to the free list at zero."""
        if self.refcount[b] <= 0:
            raise RuntimeError(f"block {b} released with refcount {self.refcount[b]}")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free_stack.append(b)

    # -- sequences --------------------------------------------------------------
    def new_seq(self) -> int:
        sid = self._next_seq
        self._next_seq += 1
        self.tables[sid] = []
        return sid

    def append(self, sid: int) -> TableEntry:
        """Append one token to sequence ``sid``; returns the entry it landed in.

        Allocates a block when the last one is full (or there is none) and
        copies a shared, partly filled last block before writing into it.
        """
        table = self.tables[sid]
        if not table or table[-1].filled == self.block_size:
            b = self.allocate()
            table.append(TableEntry(b, 0))
        last = table[-1]
        if self.refcount[last.block] > 1:
            # copy-on-write: the writer moves to a private copy
            new = self.allocate()
            self.copies.append((last.block, new))
            self.refcount[last.block] -= 1
            last = TableEntry(new, last.filled)
            table[-1] = last
        last.filled += 1
        return last

    def append_tokens(self, sid: int, n: int) -> None:
        """Append ``n`` tokens, all or nothing: raises ``PoolExhausted`` without
        changing anything when the pool cannot hold them."""
        table = self.tables[sid]
        need = 0
        room = 0
        if table:
            last = table[-1]
            room = self.block_size - last.filled
            if self.refcount[last.block] > 1 and room > 0 and n > 0:
                need += 1  # the copy-on-write block
        if n > room:
            need += -(-(n - room) // self.block_size)
        if need > self.num_free():
            raise PoolExhausted(f"sequence {sid} needs {need} blocks, {self.num_free()} free")
        for _ in range(n):
            self.append(sid)

    def fork(self, parent: int) -> int:
        """New sequence sharing every block of ``parent`` (each count + 1)."""
        child = self.new_seq()
        self.tables[child] = [TableEntry(e.block, e.filled) for e in self.tables[parent]]
        for e in self.tables[child]:
            self.refcount[e.block] += 1
        return child

    def free_seq(self, sid: int) -> None:
        for e in self.tables.pop(sid):
            self.release(e.block)

    # -- views ----------------------------------------------------------------
    def block_ids(self, sid: int) -> list:
        return [e.block for e in self.tables[sid]]

    def fills(self, sid: int) -> list:
        return [e.filled for e in self.tables[sid]]

    def check(self) -> None:
        """Invariants: counts equal the number of table references, no block is
        both free and referenced, and no count is negative."""
        refs = [0] * self.num_blocks
        for table in self.tables.values():
            for e in table:
                refs[e.block] += 1
        free = set(self.free_stack)
        if len(free) != len(self.free_stack):
            raise AssertionError("a block is on the free list twice")
        for b in range(self.num_blocks):
            if self.refcount[b] < 0:
                raise AssertionError(f"negative count on block {b}")
            if refs[b] != self.refcount[b]:
                raise AssertionError(f"block {b}: count {self.refcount[b]} != references {refs[b]}")
            if (b in free) != (refs[b] == 0):
                raise AssertionError(f"block {b}: free={b in free} references={refs[b]}")
