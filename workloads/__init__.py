"""Seeded synthetic inputs for the paged-KV decode path.

This package draws random numbers and nothing else: context lengths, the
initial free-list order of the block pool, and the query / key / value
values (rounded to the storage dtype).  It holds none of the method's
arithmetic -- no block tables, slots, copy-on-write decisions or attention --
so that the oracle and the HIP path, which both start from these inputs, share
no code beyond them.
"""
from .generators import (  # noqa: F401
    CONFIG_NAMES,
    Workload,
    make,
    make_custom,
    make_prefill,
    round_to_dtype_bits,
    bits_dtype,
)
