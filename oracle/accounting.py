"""KV-cache size and block/waste arithmetic (oracle; test infrastructure only).

* ``kv_bytes`` is the closed form of "KV Cache for the intermediate", section
  "Precise scientific definition" (the KV_size equation): two tensors (K and V)
  times layers, tokens, KV heads, head dimension and bytes per element.
* ``blocks_needed`` / ``paged_waste`` follow the 16-token blocks of
  "PagedAttention for the professional" (section "The scientific explanation"):
  only the last block of a sequence can be partly empty ("KV Cache and
  PagedAttention: why your LLM server slows down", second article, section
  "Key benefits").
* ``contiguous_waste`` is the slack of a max-length contiguous reservation
  ("PagedAttention for the professional", library-shelves section: a request
  that stops at 300 of 4096 reserved tokens leaves 3796 idle).
* ``blocks_for_bytes`` sizes a pool from a memory budget (the memory fraction
  given to the KV pool in "KV cache and PagedAttention: why the LLM server
  chokes at 10 users", serve-command section).

Pins (tests/test_oracle_accounting.py): every number the pages print for these
formulas (327,680 bytes per token for Llama 3 70B in fp16, its 32K-token total,
the MHA total, the Llama 3 8B table, ~1.3 GB per 4096-token request, 3796 idle
slots / ~93 %), plus brute-force block counting.
"""
BLOCK_SIZE = 16


def kv_bytes(num_layers: int, seq_length: int, num_kv_heads: int, head_dim: int,
             precision_bytes: int) -> int:
    return 2 * num_layers * seq_length * num_kv_heads * head_dim * precision_bytes


def blocks_needed(length: int, block_size: int = BLOCK_SIZE) -> int:
    return -(-int(length) // block_size)


def paged_waste(length: int, block_size: int = BLOCK_SIZE) -> int:
    """Empty slots of a sequence stored in whole blocks."""
    return blocks_needed(length, block_size) * block_size - int(length)


def contiguous_waste(length: int, reserved: int) -> int:
    """Empty slots of a contiguous reservation of ``reserved`` tokens."""
    if length > reserved:
        raise ValueError("sequence longer than its reservation")
    return int(reserved) - int(length)


def waste_fraction(lengths, block_size: int = BLOCK_SIZE) -> float:
    """Empty slots / allocated slots over a batch stored in whole blocks."""
    used = sum(int(n) for n in lengths)
    alloc = sum(blocks_needed(n, block_size) * block_size for n in lengths)
    return (alloc - used) / alloc if alloc else 0.0


def blocks_for_bytes(budget_bytes: int, num_layers: int, num_kv_heads: int,
                     head_dim: int, elem_bytes: int, block_size: int = BLOCK_SIZE) -> int:
    """Whole blocks (K and V of every layer) that fit in ``budget_bytes``."""
    per_block = kv_bytes(num_layers, block_size, num_kv_heads, head_dim, elem_bytes)
    return int(budget_bytes) // per_block
