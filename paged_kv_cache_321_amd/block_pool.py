"""Host-side physical block pool and per-sequence block tables.

This is bookkeeping that runs on the host; it decides which physical block a
logical block of a sequence lives in and when a shared block must be copied
before it is written.  The device work it asks for (whole-block copies) is
returned as (src, dst) pairs for ``pa_copy_blocks``.

Behaviour follows the pages' description of paged KV memory:

* "详解vLLM推理引擎架构：PagedAttention原理与LLM高效部署实践" (tbr8.org),
  section "Copy-on-Write 与内存共享": a forked table shares every block of
  its parent and raises each block's reference count; writing into a block
  whose count is above one first takes a fresh block, copies the old one into
  it, drops one reference from the old block and repoints the table entry.
* "vLLM 深度解读" (luoboask.github.io), section 2 "BlockManager": the
  allocator hands out blocks from a free set and fails loudly when the set is
  empty; a table needs ceil(tokens / block_size) blocks.

The new block's reference count is 1 (the pages leave it unset).
"""

from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple


class BlockPoolExhausted(RuntimeError):
    """Raised when a block is requested from a pool with no free blocks."""


class BlockPool:
    """A pool of ``num_blocks`` physical blocks with reference counts.

    ``order`` fixes the sequence in which free blocks are handed out (a
    seeded permutation gives shuffled physical IDs); freed blocks go to the
    back of that queue.
    """

    def __init__(self, num_blocks: int, order: Optional[Sequence[int]] = None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        order = list(range(num_blocks)) if order is None else [int(b) for b in order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self._free: List[int] = order
        self._head = 0
        self._refcount = [0] * num_blocks

    # -- allocation -------------------------------------------------------
    def num_free(self) -> int:
        return len(self._free) - self._head

    def allocate(self) -> int:
        if self._head >= len(self._free):
            raise BlockPoolExhausted("block pool exhausted: no free blocks")
        block = self._free[self._head]
        self._head += 1
        self._refcount[block] = 1
        return block

    def _release(self, block: int) -> None:
        self._free.append(block)

    # -- reference counts -------------------------------------------------
    def refcount(self, block: int) -> int:
        return self._refcount[block]

    def incref(self, block: int) -> None:
        if self._refcount[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self._refcount[block] += 1

    def decref(self, block: int) -> None:
        if self._refcount[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self._refcount[block] -= 1
        if self._refcount[block] == 0:
            self._release(block)


class BlockTable:
    """Logical-to-physical block map of one sequence."""

    def __init__(self, pool: BlockPool, block_size: int):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.pool = pool
        self.block_size = block_size
        self.blocks: List[int] = []

    @staticmethod
    def blocks_for(num_tokens: int, block_size: int) -> int:
        return -(-num_tokens // block_size)

    def append_block(self) -> int:
        block = self.pool.allocate()
        self.blocks.append(block)
        return block

    def ensure_tokens(self, num_tokens: int) -> None:
        """Allocate blocks until ``num_tokens`` tokens fit."""
        while len(self.blocks) < self.blocks_for(num_tokens, self.block_size):
            self.append_block()

    def fork(self) -> "BlockTable":
        """A new table sharing every block of this one (counts raised)."""
        child = BlockTable(self.pool, self.block_size)
        child.blocks = list(self.blocks)
        for block in child.blocks:
            self.pool.incref(block)
        return child

    def prepare_write(self, logical_block: int) -> Optional[Tuple[int, int]]:
        """Make ``logical_block`` private before a write.

        Returns the (src, dst) copy the device must perform first, or None if
        the block was already private.
        """
        old = self.blocks[logical_block]
        if self.pool.refcount(old) <= 1:
            return None
        new = self.pool.allocate()
        self.pool.decref(old)
        self.blocks[logical_block] = new
        return (old, new)

    def slot_of(self, position: int) -> int:
        """Cache slot of token ``position``: block * block_size + offset."""
        return self.blocks[position // self.block_size] * self.block_size + position % self.block_size

    def free(self) -> None:
        for block in self.blocks:
            self.pool.decref(block)
        self.blocks = []


def padded_rows(tables: Iterable[Sequence[int]], width: Optional[int] = None,
                pad: int = -1) -> List[List[int]]:
    """Block-table rows padded with ``pad`` to a common width."""
    rows = [list(t) for t in tables]
    width = max((len(r) for r in rows), default=0) if width is None else width
    if any(len(r) > width for r in rows):
        raise ValueError("a table is wider than the requested width")
    return [r + [pad] * (width - len(r)) for r in rows]


def prefix_groups(rows: Sequence[Sequence[int]], context_lens: Sequence[int],
                  block_size: int) -> Tuple[List[int], List[int]]:
    """Groups of consecutive sequences whose tables start with the same blocks.

    Beams forked from one sequence, or requests that reuse one cached prompt,
    name the same physical blocks in their leading table entries ("Copy-on-Write
    与内存共享" and "Prefix Caching（前缀缓存）" on the tbr8.org page).  Returns
    ``(leader, blocks)`` for ``pa_decode_shared_prefix``: ``leader[s]`` is the
    first sequence of s's group, and at a leader ``blocks[L]`` is the number of
    leading entries every member holds in common, counting only blocks that are
    full for every member (``blocks * block_size <= context_len``).  A sequence
    joins the group before it when it shares at least one such block with the
    group's leader; other entries of ``blocks`` are 0.
    """
    n = len(rows)
    leader = list(range(n))
    blocks = [0] * n
    lead = -1
    for s in range(n):
        full = int(context_lens[s]) // block_size
        if lead >= 0:
            limit = min(blocks[lead], full)
            common = 0
            while common < limit and rows[s][common] == rows[lead][common]:
                common += 1
            if common > 0:
                leader[s] = lead
                blocks[lead] = common
                continue
        lead = s
        blocks[s] = full
    # A leader without members shares nothing.
    members = {leader[s] for s in range(n) if leader[s] != s}
    for s in range(n):
        if leader[s] == s and s not in members:
            blocks[s] = 0
    return leader, blocks


def prefix_bounds(leader: Sequence[int], blocks: Sequence[int], context_lens: Sequence[int],
                  block_size: int) -> Tuple[int, int]:
    """Host bounds (max_prefix_blocks, max_tail_len) for a well-formed grouping.

    ``leader``/``blocks`` as returned by ``prefix_groups``: every sequence's
    shared prefix is its leader's block count, and its tail is the rest of its
    context (the whole context when it shares nothing).
    """
    max_blocks = 0
    max_tail = 0
    for s, c in enumerate(context_lens):
        lead = leader[s]
        n = blocks[lead] if (leader[lead] == lead and blocks[lead] > 0) else 0
        max_blocks = max(max_blocks, n)
        max_tail = max(max_tail, int(c) - n * block_size)
    return max_blocks, max_tail
