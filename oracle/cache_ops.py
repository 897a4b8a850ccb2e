"""Reference cache writes and block copies (oracle; test infrastructure only).

The oracle's cache is the logical view ``[num_blocks, num_kv_heads, 16, head_dim]``
of stored bits: slot ``b*16 + i`` is row ``i`` of block ``b``.  Only the new
token's K and V are written each step; everything older is read back from the
cache ("KV Cache and PagedAttention: why your LLM server slows down", second
article, section "What is the KV cache?").  A block copy duplicates a shared
block before one sharer writes into it (same page, section "How PagedAttention
fixes this": shared prefixes with copy-on-write).

Pins (tests/test_oracle_cache_ops.py): hand-written expected arrays on tiny
caches, the -1 "skip" slot, copy-before-write ordering of a shared partial
block, and untouched slots keeping their bits.
"""
import numpy as np

BLOCK_SIZE = 16


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping) -> None:
    """k_cache[slot // 16, :, slot % 16, :] = key[t] (and V alike); slot -1 skips."""
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, row = divmod(int(slot), BLOCK_SIZE)
        k_cache[block, :, row, :] = key[t]
        v_cache[block, :, row, :] = value[t]


def copy_blocks(k_cache, v_cache, pairs) -> None:
    """For each (src, dst) in order: block dst of K and V becomes block src."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def transfer_blocks(src_k, src_v, dst_k, dst_v, pairs) -> None:
    """For each (s, d): block d of the destination caches becomes block s of
    the source caches (the data side of moving blocks between tiers)."""
    for s, d in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        dst_k[d] = src_k[s]
        dst_v[d] = src_v[s]
