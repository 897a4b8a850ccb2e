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

Readings where the pages leave a step open:
* the pool is a stack seeded from ``free_order``: the first ``alloc`` returns
  ``free_order[0]``; a block whose count drops to 0 is pushed back and is the
  next one handed out (in the shelves example a returned shelf is reused
  right away);
* blocks of one append are taken in logical order; a copy-on-write destination
  is taken before any fresh block of the same append;
* a write into a block whose reference count is above 1 copies it first, the
  writer gets the copy and the source loses one reference; a block at count 1
  is written in place (so of n sharers, the first n-1 writers copy).

Prefix caching: blocks are reused when several requests start with the same
tokens, e.g. one system prompt ("PagedAttention for the professional", the
serve-command section on --enable-prefix-caching), and the cached blocks
consume room in the pool (same page, trade-offs section).  Readings:
* only full blocks are cached; a block's key is (the serial number of the
  entry of the block before it, or 0 for the first block; its 16 token ids).
  Serial numbers are never reused, so a key names a whole token prefix
  exactly -- no hashing, no collisions -- and an entry whose parent was
  evicted simply becomes unreachable;
* ``register`` enters the full blocks of a sequence's table; a block whose key
  is already cached under another block is left out (the chain continues
  through the cached entry, which holds the same prefix);
* ``match_prefix`` walks the key chain of a token list from the first block
  and takes one reference on every cached block it finds, stopping at the
  first miss;
* a cached block whose count drops to 0 stays cached and joins the end of an
  eviction list; allocation takes an uncached free block first (LIFO as
  above) and only then evicts the least recently released cached block.

Host tier (swapping): when the device pool runs short, individual blocks can
move to a pool in host memory instead of whole sequences ("KV Cache and
PagedAttention: why your LLM server slows down", the contrast between
all-or-nothing eviction of a whole sequence to the CPU and fine-grained
eviction of small pages).  Readings: the host tier is a second BlockPool of
the same block shape; ``swap_blocks`` moves a list of blocks from one pool to
the other -- each gets a fresh block in the destination (taken in list order,
before anything is released), the (source, destination) pairs are what the
device must copy, and the source block loses the one reference that moved
(a block still shared by others stays where it is for them).  All or
nothing.

Pins (tests/test_oracle_pool.py): the pages' worked examples (token 17 -> second
block; 300 of a 4096 reservation idle), block count = ceil(len/16) with waste
below 16 slots per sequence, reference-count conservation against the tables
after random operation sequences, LIFO reuse, all-or-nothing failure, and the
shared-prefix workload's closed-form copy count and block count.  Prefix
caching (tests/test_oracle_prefix.py): matched blocks = floor(common prefix /
16) by brute force over random token lists, cached blocks outliving their
sequences, eviction order, no false hit through a reused block id, and the
shared-prompt block count in closed form.  Swapping (tests/test_oracle_swap.py):
references conserved across both tiers, a swap out and back in restores every
sequence's K/V bits and decode output exactly, shared blocks stay for the other
sharers, all-or-nothing failure, and the page's fine-grained versus
whole-sequence eviction counts.
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
        # prefix cache
        self.cache = {}        # key -> block
        self.key_of = {}       # block -> key
        self.serial_of = {}    # block -> serial number of its entry
        self.next_serial = 1
        self.lru = []          # cached blocks at count 0, least recently released first
        self.prefix_hits = 0

    # -- single-block calls --
    def num_free(self) -> int:
        """Blocks an allocation can take: uncached free ones and evictable ones."""
        return len(self.free_stack) + len(self.lru)

    def _check(self, b: int) -> int:
        b = int(b)
        if not 0 <= b < self.num_blocks or self.refcount[b] == 0:
            raise BadBlock(f"block {b} is not held")
        return b

    def alloc(self) -> int:
        if self.free_stack:
            b = self.free_stack.pop()
        elif self.lru:
            b = self.lru.pop(0)
            self._uncache(b)
        else:
            raise OutOfBlocks("pool is empty")
        self.refcount[b] = 1
        return b

    def _chain_id(self, b: int) -> int:
        """What the key of the block after cached block ``b`` names as its
        parent: the serial number of b's entry."""
        return self.serial_of[b]

    def _uncache(self, b: int) -> None:
        del self.cache[self.key_of.pop(b)]
        del self.serial_of[b]

    def incref(self, b: int) -> None:
        b = self._check(b)
        self.refcount[b] += 1

    def free(self, b: int) -> None:
        """Drop one reference; at zero the block goes back on top of the pool."""
        b = self._check(b)
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            if b in self.key_of:
                self.lru.append(b)
            else:
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

    # -- prefix cache --
    @staticmethod
    def _full_blocks(tokens):
        tokens = [int(t) for t in tokens]
        return [tuple(tokens[i:i + BLOCK_SIZE])
                for i in range(0, len(tokens) - BLOCK_SIZE + 1, BLOCK_SIZE)]

    def match_prefix(self, tokens) -> list:
        """Cached blocks holding the longest run of whole leading blocks of
        ``tokens``; each gets one more reference (the caller's new table)."""
        found = []
        parent = 0
        for chunk in self._full_blocks(tokens):
            b = self.cache.get((parent, chunk))
            if b is None:
                break
            found.append(b)
            parent = self._chain_id(b)
        for b in found:
            if self.refcount[b] == 0:
                self.lru.remove(b)
            self.refcount[b] += 1
        self.prefix_hits += len(found)
        return found

    def register(self, table, tokens) -> int:
        """Cache the full blocks of a sequence whose first tokens are
        ``tokens`` and whose blocks are ``table``.  Returns how many blocks
        were entered.  All-or-nothing: every block must be held and a block
        already cached must hold the same 16 tokens."""
        chunks = self._full_blocks(tokens)
        if len(chunks) > len(table):
            raise InvalidArg("more full blocks of tokens than table entries")
        for i, chunk in enumerate(chunks):
            b = self._check(table[i])
            if b in self.key_of and self.key_of[b][1] != chunk:
                raise InvalidArg(f"block {b} is cached with other tokens")
        added = 0
        parent = 0
        for i, chunk in enumerate(chunks):
            b = int(table[i])
            if b not in self.key_of:
                other = self.cache.get((parent, chunk))
                if other is not None:
                    parent = self._chain_id(other)
                    continue
                self.cache[(parent, chunk)] = b
                self.key_of[b] = (parent, chunk)
                self.serial_of[b] = self.next_serial
                self.next_serial += 1
                added += 1
            parent = self._chain_id(b)
        return added

    # -- accounting --
    def stats(self) -> dict:
        used = sum(1 for r in self.refcount if r > 0)
        shared = sum(1 for r in self.refcount if r > 1)
        return {"num_blocks": self.num_blocks, "free": self.num_free(), "used": used,
                "shared": shared, "copies": self.copies_made, "cached": len(self.key_of),
                "evictable": len(self.lru), "prefix_hits": self.prefix_hits}


def swap_blocks(src: BlockPool, dst: BlockPool, blocks) -> list:
    """Move ``blocks`` (ids held in ``src``) to ``dst``: returns the
    (src_block, dst_block) pairs to copy, in list order; the caller's table
    entries become the dst blocks.  All or nothing."""
    blocks = [int(b) for b in blocks]
    for b in set(blocks):  # one held reference per listing
        if not 0 <= b < src.num_blocks or src.refcount[b] < blocks.count(b):
            raise BadBlock(f"block {b} is not held often enough")
    if dst.num_free() < len(blocks):
        raise OutOfBlocks("destination pool cannot take these blocks")
    pairs = [(b, dst.alloc()) for b in blocks]
    for b in blocks:
        src.free(b)
    return pairs
