"""Oracle for the paged-KV decode path: plain, slow, CPU, float64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything here: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``paged_kv_cache_06_amd``); both start from the seeded inputs of
``workloads`` and nothing else.

What it computes, and where the pages define it
-----------------------------------------------
* ``pool``      -- the block pool: fixed 16-token blocks handed out on demand,
                   returned on free, shared by reference count, copied on write.
                   ("PagedAttention for the professional", sections "Beginner's
                   example: library shelves" and "The scientific explanation";
                   "KV Cache and PagedAttention: why your LLM server slows
                   down", sections "How PagedAttention fixes this" and "How does
                   PagedAttention work?")
* ``cache_ops`` -- writing new tokens' K/V into their slots, copying blocks.
* ``attention`` -- decode attention of one new query per head against every
                   cached K/V of the sequence, with grouped-query heads
                   ("KV Cache for the intermediate", sections "Precise scientific
                   definition" and "Grouped Query Attention").  The pages name
                   the attention dot product but print no formula; the oracle
                   takes textbook scaled dot-product softmax attention.
* ``accounting``-- the KV-size closed form and the block/waste arithmetic
                   ("KV Cache for the intermediate", section "Precise scientific
                   definition", the KV_size equation and its worked example).
* ``quant``     -- the INT8 cache: per-channel symmetric codes, and decode
                   attention over the values they stand for ("KV Cache for the
                   intermediate", section "KV Cache Quantization").
* ``step``      -- the order in which a batch is prefilled and stepped, built
                   from the calls above.

Every function is pinned by ``tests/test_oracle_*.py`` against values the pages
print, closed forms, brute force on tiny inputs, a library routine and
invariants; see the header of each module for the pins that cover it.
"""
from . import accounting, attention, cache_ops, numerics, pool, quant, step  # noqa: F401
