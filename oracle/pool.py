"""Reference block pool (oracle; test infrastructure only).

The KV cache is cut into fixed blocks of 16 token slots that can sit anywhere in
one pool; each sequence keeps a table from its logical blocks to physical ones,
and a new block is taken only when the sequence needs another slot -- token 17
opens the second block ("PagedAttention for the professional", sections
"Beginner's example: library shelves" and "The scientific explanation"; "What
PagedAttention is and what it changed in LLM serving", section "PagedAttention
simply").  A finished sequence's blocks go straight back to the pool for the
next request (same page, library-shelves section).  Several sequences may map
the same physical blocks of a common prompt, and a shared block is copied when
one of them writes into it ("KV Cache and PagedAttention: why your LLM server
slows down", section "How PagedAttention fixes this"; "PagedAttention for the
professional", results list: parallel sampling with n=4 costs about the memory
of n=1).

Readings where the pages leave a step open (listed in the design doc):
* the pool is a stack seeded from ``free_order``: the first ``alloc`` returns
  ``free_order[0]``; a block whose count drops to 0 is pushed back and is the
  next one handed out (in the shelves example a returned shelf is reused
  right away);
* blocks of one append are taken in logical order; a copy-on-write destination
  is taken before any fresh block of the same append;
* a write into a block whose reference count is above 1 copies it first, the
  writer gets the copy and the source loses one reference; a block at count 1
  is written in place (so of n sharers, the first n-1 writers copy).

Pins (tests/test_oracle_pool.py): the pages' worked examples (token 17 -> second
block; 300 of a 4096 reservation idle), block count = ceil(len/16) with waste
below 16 slots per sequence, reference-count conservation against the tables
after random operation sequences, LIFO reuse, all-or-nothing failure, and the
shared-prefix workload's closed-form copy count and block count.
"""
from __future__ import annotations

BLOCK_SIZE = 16


class PoolError(Exception):
    pass


class OutOfBlocks(PoolError):
    pass


class BadBlock(PoolError):
    pass


class InvalidArg(PoolError):
    pass


def blocks_for(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Blocks that hold ``num_tokens`` tokens: ceil(num_tokens / block_size)."""
    return -(-int(num_tokens) // block_size)


class BlockPool:
    def __init__(self, num_blocks: int, free_order=None):
        num_blocks = int(num_blocks)
        if num_blocks <= 0:
            raise InvalidArg("pool needs at least one block")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.refcount = [0] * num_blocks
        self.free_stack = list(reversed(order))  # top of the stack = order[0]
        self.copies_made = 0

    # -- single-block calls --
    def num_free(self) -> int:
        return len(self.free_stack)

    def _check(self, b: int) -> int:
        b = int(b)
        if not 0 <= b < self.num_blocks or self.refcount[b] == 0:
            raise BadBlock(f"block {b} is not held")
        return b

    def alloc(self) -> int:
        if not self.free_stack:
            raise OutOfBlocks("pool is empty")
        b = self.free_stack.pop()
        self.refcount[b] = 1
        return b

    def incref(self, b: int) -> None:
        b = self._check(b)
        self.refcount[b] += 1

    def free(self, b: int) -> None:
        """Drop one reference; at zero the block goes back on top of the pool."""
        b = self._check(b)
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free_stack.append(b)

    # -- whole-table calls --
    def fork(self, table) -> list:
        """A new sequence that shares every block of ``table``."""
        for b in table:
            self._check(b)
        for b in table:
            self.refcount[b] += 1
        return list(table)

    def free_table(self, table) -> None:
        for b in table:
            self.free(b)
        del table[:]

    def append(self, table: list, pos: int, n: int, max_blocks: int | None = None):
        """Give ``n`` new tokens at positions pos..pos+n-1 their slots.

        ``table`` must hold exactly the blocks of the first ``pos`` tokens.
        Returns (slots, cow) where slot = physical_block * 16 + position % 16
        and cow is the (source, destination) block pair of a copy-on-write, or
        None.  On failure nothing changes.
        """
        pos, n = int(pos), int(n)
        if pos < 0 or n < 0 or len(table) != blocks_for(pos):
            raise InvalidArg("table does not match the position")
        if n == 0:
            return [], None
        after = blocks_for(pos + n)
        if max_blocks is not None and after > max_blocks:
            raise InvalidArg("table row is full")
        fresh = after - len(table)
        cow_needed = pos % BLOCK_SIZE != 0 and self.refcount[table[pos // BLOCK_SIZE]] > 1
        if self.num_free() < fresh + int(cow_needed):
            raise OutOfBlocks("not enough free blocks for this append")
        cow = None
        if cow_needed:
            src = table[pos // BLOCK_SIZE]
            dst = self.alloc()
            self.free(src)  # count > 1 before, so src stays held by the others
            table[pos // BLOCK_SIZE] = dst
            cow = (src, dst)
            self.copies_made += 1
        for _ in range(fresh):
            table.append(self.alloc())
        slots = []
        for p in range(pos, pos + n):
            slots.append(table[p // BLOCK_SIZE] * BLOCK_SIZE + p % BLOCK_SIZE)
        return slots, cow

    # -- accounting --
    def stats(self) -> dict:
        used = sum(1 for r in self.refcount if r > 0)
        shared = sum(1 for r in self.refcount if r > 1)
        return {"num_blocks": self.num_blocks, "free": self.num_free(), "used": used,
                "shared": shared, "copies": self.copies_made}
