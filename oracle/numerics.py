"""Exact conversion of stored bits to float64 (oracle; test infrastructure only).

bf16 is the top half of an IEEE binary32; fp16 is IEEE binary16.  Both widen to
float64 exactly.  Pinned in tests/test_oracle_numerics.py against Python's own
``struct`` decoding of the same bit patterns.
"""
import numpy as np


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Stored bits of ``dtype`` ("f32", "bf16", "f16") -> float64, exactly."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.float32, copy=False).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16, copy=False).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        wide = bits.astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
