"""Host-side physical block pool and per-sequence block tables.

This is the allocator half of PagedAttention: the device never sees it, it only
receives the int32 block tables it produces.

Sources (the pages describe the structures, they ship no allocator):
  * 5688vip.com "vLLM核心机制" §3.1 -- logical blocks map through a per-request
    table to non-contiguous physical blocks; a new block is appended when the
    last one fills; finished requests return their blocks to the free pool;
    requests that share a prefix share its physical blocks.
  * gaoleia.github.io "PagedAttention 和 Continuous Batching" §1.3 (a block
    carries num_tokens 0..block_size and a ref_count) and §1.4 (BlockTable:
    mapping list, get_physical_block, append_block).
  * feifeigd.github.io "vLLM 架构详解" 一 PagedAttention, "Block Table 实现" and
    "共享前缀的 Block 复用" (ref-counted sharing: A=[B0..B4], B=[B0..B3,B5]
    leaves B0..B3 at ref 2).  That page counts a table's tokens as
    len(blocks)*block_size, which overstates the fill of the last block; here
    every table tracks its true token count instead (the num_tokens field of
    §1.3 on the gaoleia page).
  * lakecityint.com/news/209622 §4.2 (BlockManager.allocate_block pops a free
    block; exhaustion is the preemption trigger), §3.2 (copy-on-write: a
    sharer about to write gets a new block, the shared block's content is
    copied into it, its table is remapped and the old block loses one
    reference) and §2.1 (preempted sequences wait in a swapped queue with
    their blocks in CPU memory); 5688vip.com §3.3 (preemption swaps out to
    CPU or releases the blocks and recomputes later).
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple


class BlockPool:
    """Fixed pool of ``num_blocks`` physical block ids with reference counts.

    ``order`` fixes the free-list order (the first id is handed out first); a
    seeded permutation gives the shuffled placement the workloads use.  Ids are
    returned to the back of the free list when their count drops to zero.
    """

    def __init__(self, num_blocks: int, order: Optional[Iterable[int]] = None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        self.num_blocks = int(num_blocks)
        free = list(range(self.num_blocks)) if order is None else [int(b) for b in order]
        if sorted(free) != list(range(self.num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self._free: List[int] = free
        self._head = 0
        self._ref = [0] * self.num_blocks

    # -- queries --------------------------------------------------------
    def num_free(self) -> int:
        return len(self._free) - self._head

    def ref_count(self, block: int) -> int:
        return self._ref[block]

    def ref_counts(self) -> List[int]:
        return list(self._ref)

    # -- mutation -------------------------------------------------------
    def alloc(self) -> int:
        """Pop a free block with ref_count 1; raises MemoryError when empty."""
        if self._head >= len(self._free):
            raise MemoryError("block pool exhausted (%d blocks)" % self.num_blocks)
        b = self._free[self._head]
        self._head += 1
        if self._head > 4096 and self._head * 2 > len(self._free):
            del self._free[: self._head]
            self._head = 0
        self._ref[b] = 1
        return b

    def incref(self, block: int) -> None:
        if self._ref[block] <= 0:
            raise ValueError("incref of a free block %d" % block)
        self._ref[block] += 1

    def free(self, block: int) -> None:
        """Drop one reference; the block returns to the free list at zero."""
        if self._ref[block] <= 0:
            raise ValueError("double free of block %d" % block)
        self._ref[block] -= 1
        if self._ref[block] == 0:
            self._free.append(block)


class SeqBlocks:
    """One sequence's block table: logical block i lives in physical block
    ``mapping[i]``; ``num_tokens`` is the exact number of tokens it holds."""

    def __init__(self, block_size: int):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.block_size = int(block_size)
        self.mapping: List[int] = []
        self.num_tokens = 0

    def get_physical_block(self, logical_idx: int) -> int:
        return self.mapping[logical_idx]

    def append_block(self, physical_block: int) -> None:
        self.mapping.append(int(physical_block))

    def append_tokens(self, n: int, pool: BlockPool) -> None:
        """Make room for ``n`` more tokens, allocating blocks on demand."""
        if n < 0:
            raise ValueError("n must be >= 0")
        total = self.num_tokens + n
        need = -(-total // self.block_size)
        while len(self.mapping) < need:
            self.append_block(pool.alloc())
        self.num_tokens = total

    def share_prefix_from(self, other: "SeqBlocks", n_blocks: int, pool: BlockPool) -> None:
        """Start this (empty) table with ``other``'s first ``n_blocks`` full
        blocks, taking one reference on each."""
        if self.mapping:
            raise ValueError("share_prefix_from needs an empty table")
        if n_blocks > len(other.mapping) or n_blocks * self.block_size > other.num_tokens:
            raise ValueError("other does not hold %d full blocks" % n_blocks)
        if other.block_size != self.block_size:
            raise ValueError("block sizes differ")
        for b in other.mapping[:n_blocks]:
            pool.incref(b)
            self.append_block(b)
        self.num_tokens = n_blocks * self.block_size

    def fork(self, pool: BlockPool) -> "SeqBlocks":
        """A new table sharing every block of this one, including a partly
        filled last block (parallel sampling from one prompt)."""
        child = SeqBlocks(self.block_size)
        for b in self.mapping:
            pool.incref(b)
            child.append_block(b)
        child.num_tokens = self.num_tokens
        return child

    def prepare_write(self, logical_idx: int, pool: BlockPool) -> Optional[Tuple[int, int]]:
        """Copy-on-write before writing into logical block ``logical_idx``: a
        block other tables still reference is replaced by a fresh block that
        must receive a copy of it.  Returns (old, new) for the device copy, or
        None when the block is already private."""
        old = self.mapping[logical_idx]
        if pool.ref_count(old) <= 1:
            return None
        new = pool.alloc()
        self.mapping[logical_idx] = new
        pool.free(old)                       # drop this table's reference
        return old, new

    def prepare_append(self, n: int, pool: BlockPool) -> List[Tuple[int, int]]:
        """Room for ``n`` more tokens, copying a shared partly filled last
        block first; returns the (old, new) copies the device must make."""
        copies = []
        if n > 0 and self.mapping and self.num_tokens % self.block_size:
            cw = self.prepare_write(len(self.mapping) - 1, pool)
            if cw:
                copies.append(cw)
        self.append_tokens(n, pool)
        return copies

    def release(self, pool: BlockPool) -> None:
        for b in self.mapping:
            pool.free(b)
        self.mapping = []
        self.num_tokens = 0

    def row(self, width: int) -> List[int]:
        """The table padded with -1 to ``width`` entries (device row format)."""
        if width < len(self.mapping):
            raise ValueError("width %d < %d blocks" % (width, len(self.mapping)))
        return self.mapping + [-1] * (width - len(self.mapping))


def tables_to_rows(tables: Sequence[SeqBlocks], width: Optional[int] = None) -> List[List[int]]:
    w = max((len(t.mapping) for t in tables), default=0) if width is None else width
    w = max(w, 1)
    return [t.row(w) for t in tables]


def swap_out(table: SeqBlocks, gpu_pool: BlockPool, cpu_pool: BlockPool) -> List[Tuple[int, int]]:
    """Move a table's blocks to CPU blocks: returns (gpu, cpu) copies to make
    before the GPU blocks are reused; the table then holds CPU ids.  A block
    other tables share stays on the GPU for them (only a reference is
    dropped) and this table gets its own CPU copy.  Raises MemoryError, and
    changes nothing, when the CPU pool lacks room."""
    if cpu_pool.num_free() < len(table.mapping):
        raise MemoryError("CPU pool has %d free blocks, %d needed" % (cpu_pool.num_free(), len(table.mapping)))
    pairs = []
    for i, b in enumerate(table.mapping):
        c = cpu_pool.alloc()
        pairs.append((b, c))
        gpu_pool.free(b)
        table.mapping[i] = c
    return pairs


def swap_in(table: SeqBlocks, cpu_pool: BlockPool, gpu_pool: BlockPool) -> List[Tuple[int, int]]:
    """Bring a swapped table back: returns (cpu, gpu) copies; the CPU blocks
    are free again once the copies are done.  Raises MemoryError, and changes
    nothing, when the GPU pool lacks room."""
    if gpu_pool.num_free() < len(table.mapping):
        raise MemoryError("GPU pool has %d free blocks, %d needed" % (gpu_pool.num_free(), len(table.mapping)))
    pairs = []
    for i, c in enumerate(table.mapping):
        g = gpu_pool.alloc()
        pairs.append((c, g))
        cpu_pool.free(c)
        table.mapping[i] = g
    return pairs
