"""INT8 KV cache with per-channel scales (oracle; test infrastructure only).

K and V may be stored as 8-bit integers instead of 16-bit floats, which halves
the cache, and per-channel scales keep the quality loss small ("KV Cache for
the intermediate", section "KV Cache Quantization"; the same page's trade-offs
list the extra dequantization latency, and its next-step list says to try INT8
before INT4).

Readings where the page leaves the scheme open:
* symmetric quantization with one fp32 scale s > 0 per (KV head, channel),
  one scale array for K and one for V, supplied by the caller (calibration is
  the caller's business);
* code = clamp(round-half-even(x / s), -127, 127) where x is the stored
  16-bit value widened exactly to fp32 and x / s is one IEEE fp32 division:
  the integer decision is taken in fp32, so both implementations take it
  identically.  NaN quantizes to 0, +-inf to +-127; -128 is never produced;
* the cache then holds the values code * s (exact in float64), and decode
  attention is the unquantized oracle's attention over exactly those values.

Pins (tests/test_oracle_quant.py): the code equals the nearest integer of the
exact rational x / s (Python fractions) wherever that is not within fp32
rounding of a tie; ties go to even; saturation, infinities, NaN and sign
symmetry; |code * s - x| <= s / 2 on the representable range; values that are
exact multiples code * s round-trip exactly, and decode over such a cache
equals the unquantized oracle's decode bit for bit (per-head, per-channel
power-of-two scales, which also pins the scale indexing).
"""
import numpy as np

from .attention import BLOCK_SIZE, attend
from .numerics import to_f64

CODE_MAX = 127


def quantize(bits, dtype: str, scale) -> np.ndarray:
    """int8 codes of stored values ``bits`` [..., Hkv, D] with scales [Hkv, D]."""
    x = to_f64(bits, dtype).astype(np.float32)  # exact: 16-bit and fp32 values fit fp32
    s = np.asarray(scale, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.rint(x / s)  # fp32 division, round half to even
    y = np.where(np.isnan(y), np.float32(0), y)
    return np.clip(y, -CODE_MAX, CODE_MAX).astype(np.int8)


def dequantize(codes, scale) -> np.ndarray:
    """The values a code array stands for, float64: code * s."""
    return np.asarray(codes).astype(np.float64) * np.asarray(scale, dtype=np.float32).astype(np.float64)


def reshape_and_cache(key_bits, value_bits, dtype: str, k_codes, v_codes, slot_mapping,
                      k_scale, v_scale) -> None:
    """Quantize the new tokens' K and V and write the codes into their slots
    (logical view [NB, Hkv, 16, D]); slot -1 skips."""
    kq = quantize(key_bits, dtype, k_scale)
    vq = quantize(value_bits, dtype, v_scale)
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, row = divmod(int(slot), BLOCK_SIZE)
        k_codes[block, :, row, :] = kq[t]
        v_codes[block, :, row, :] = vq[t]


def paged_decode(q_bits, k_codes, v_codes, k_scale, v_scale, block_tables, context_lens,
                 scale: float, dtype: str) -> np.ndarray:
    """Decode attention over an INT8 cache: out[s, h] = attention(q[s, h],
    code_K * s_K, code_V * s_V) over the sequence's positions, gathered
    through its table.  float64 [S, Hq, D]."""
    S, Hq, D = q_bits.shape
    Hkv = k_codes.shape[1]
    group = Hq // Hkv
    q = to_f64(q_bits, dtype)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        length = int(context_lens[s])
        if length == 0:
            continue
        pos = np.arange(length)
        blocks = np.asarray(block_tables[s], dtype=np.int64)[pos // BLOCK_SIZE]
        for g in range(Hkv):
            K = dequantize(k_codes[blocks, g, pos % BLOCK_SIZE, :], np.asarray(k_scale)[g])
            V = dequantize(v_codes[blocks, g, pos % BLOCK_SIZE, :], np.asarray(v_scale)[g])
            for h in range(g * group, (g + 1) * group):
                out[s, h] = attend(q[s, h], K, V, scale)
    return out
