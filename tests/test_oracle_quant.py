"""Pins of oracle.quant (INT8 KV cache) against exact arithmetic and the
unquantized oracle."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import accounting, attention, quant
from oracle.numerics import to_f64
from workloads import round_to_dtype_bits


def _exact_code(x: float, s: float):
    """Nearest integer of the exact rational x / s (ties: both neighbours),
    clamped to [-127, 127]."""
    r = Fraction(x) / Fraction(s)
    lo = r.numerator // r.denominator
    frac = r - lo
    if frac == Fraction(1, 2):
        cands = {lo, lo + 1}
    else:
        cands = {lo if frac < Fraction(1, 2) else lo + 1}
    return {max(-127, min(127, c)) for c in cands}, r


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_codes_are_the_nearest_integer_of_the_exact_ratio(dtype):
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4000).astype(np.float32) * rng.choice([0.01, 1.0, 30.0], 4000)
    bits = round_to_dtype_bits(x, dtype)
    s = rng.uniform(0.001, 0.2, 4000).astype(np.float32)
    codes = quant.quantize(bits[:, None, None], dtype, s[:, None, None]).ravel()
    xv = to_f64(bits, dtype)
    for i in range(len(xv)):
        cands, r = _exact_code(float(xv[i]), float(s[i]))
        # fp32 division is correctly rounded: away from a tie the rounding of
        # x / s cannot change the nearest integer
        near_tie = abs(abs(r - int(r)) - Fraction(1, 2)) < Fraction(1, 1 << 16) * max(1, abs(r))
        if not near_tie:
            assert int(codes[i]) in cands, (xv[i], s[i], codes[i], float(r))
        else:
            lo = int(np.floor(float(r)))
            assert int(codes[i]) in {max(-127, min(127, lo)), max(-127, min(127, lo + 1))}


def test_ties_go_to_even_and_sign_is_symmetric():
    s = np.float32(2.0 ** -5)  # x / s is exact for these x
    xs = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 126.5, -126.5], np.float32) * s
    codes = quant.quantize(xs.reshape(-1, 1, 1), "f32", np.full((1, 1), s, np.float32)).ravel()
    assert codes.tolist() == [0, 2, 2, 4, 0, -2, -2, 126, -126]
    rng = np.random.default_rng(1)
    x = round_to_dtype_bits(rng.standard_normal(2000).astype(np.float32) * 3, "bf16")
    sc = np.full((1, 1), 0.0371, np.float32)
    a = quant.quantize(x.reshape(-1, 1, 1), "bf16", sc)
    b = quant.quantize((x ^ np.uint16(0x8000)).reshape(-1, 1, 1), "bf16", sc)
    assert np.array_equal(a, -b)


def test_saturation_infinities_nan_and_no_minus_128():
    s = np.full((1, 1), 0.5, np.float32)
    x = np.array([1000.0, -1000.0, 63.5, 63.75, -63.75, np.inf, -np.inf, np.nan], np.float32)
    codes = quant.quantize(x.reshape(-1, 1, 1), "f32", s).ravel()
    assert codes.tolist() == [127, -127, 127, 127, -127, 127, -127, 0]
    rng = np.random.default_rng(2)
    many = quant.quantize(rng.standard_normal((5000, 1, 1)).astype(np.float32) * 100, "f32", s)
    assert many.min() == -127 and many.max() == 127


def test_round_trip_error_is_at_most_half_a_step():
    rng = np.random.default_rng(3)
    s = rng.uniform(0.01, 0.1, (4, 64)).astype(np.float32)
    x = (rng.uniform(-1, 1, (300, 4, 64)) * 127 * s).astype(np.float32)
    codes = quant.quantize(x, "f32", s)
    err = np.abs(quant.dequantize(codes, s) - x.astype(np.float64))
    # half a step, plus the fp32 rounding of x / s (at most 127 * 2^-24 steps)
    assert np.all(err <= s.astype(np.float64) * (0.5 + 127 * 2.0 ** -24))


def _exact_multiples(rng, shape, scale, dtype):
    """Values code * s that the storage dtype holds exactly."""
    codes = rng.integers(-127, 128, shape).astype(np.int8)
    vals = codes.astype(np.float64) * scale.astype(np.float64)
    bits = round_to_dtype_bits(vals.astype(np.float32), dtype)
    assert np.array_equal(to_f64(bits, dtype), vals)
    return codes, bits


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_exact_multiples_round_trip_and_decode_equals_the_unquantized_oracle(dtype):
    rng = np.random.default_rng(4)
    S, Hq, Hkv, D, NB = 3, 8, 2, 32, 12
    # a different power-of-two scale per (KV head, channel)
    sk = (2.0 ** -rng.integers(4, 9, (Hkv, D))).astype(np.float32)
    sv = (2.0 ** -rng.integers(4, 9, (Hkv, D))).astype(np.float32)
    kc, kb = _exact_multiples(rng, (NB, Hkv, 16, D), sk[None, :, None, :], dtype)
    vc, vb = _exact_multiples(rng, (NB, Hkv, 16, D), sv[None, :, None, :], dtype)
    assert np.array_equal(quant.quantize(kb.transpose(0, 2, 1, 3), dtype, sk),
                          kc.transpose(0, 2, 1, 3))
    assert np.array_equal(quant.quantize(vb.transpose(0, 2, 1, 3), dtype, sv),
                          vc.transpose(0, 2, 1, 3))
    q = round_to_dtype_bits(rng.standard_normal((S, Hq, D)).astype(np.float32), dtype)
    tables = np.array([rng.permutation(NB)[:4] for _ in range(S)])
    lens = np.array([1, 37, 64])
    want = attention.paged_decode(q, kb, vb, tables, lens, 0.2, dtype)
    got = quant.paged_decode(q, kc, vc, sk, sv, tables, lens, 0.2, dtype)
    assert np.array_equal(got, want)
    # the scales are indexed [KV head, channel]: swapping the heads' scales moves the result
    bad = quant.paged_decode(q, kc, vc, sk[::-1], sv, tables, lens, 0.2, dtype)
    assert not np.allclose(bad, want)


def test_reshape_and_cache_writes_codes_to_the_slots():
    rng = np.random.default_rng(6)
    Hkv, D = 2, 16
    s = rng.uniform(0.02, 0.05, (Hkv, D)).astype(np.float32)
    key = round_to_dtype_bits(rng.standard_normal((3, Hkv, D)).astype(np.float32), "bf16")
    val = round_to_dtype_bits(rng.standard_normal((3, Hkv, D)).astype(np.float32), "bf16")
    kc = np.full((4, Hkv, 16, D), 99, np.int8)
    vc = kc.copy()
    quant.reshape_and_cache(key, val, "bf16", kc, vc, [5, -1, 49], s, s)
    assert np.array_equal(kc[0, :, 5], quant.quantize(key[0], "bf16", s))
    assert np.array_equal(vc[3, :, 1], quant.quantize(val[2], "bf16", s))
    assert (kc == 99).sum() == kc.size - 2 * Hkv * D


def test_int8_halves_the_kv_bytes_per_token():
    """The page's 2x (INT8) and 4x (INT4) savings against FP16, through the
    KV_size closed form for Llama 3 70B (80 layers, 8 KV heads, D 128)."""
    fp16 = accounting.kv_bytes(80, 1, 8, 128, 2)
    assert fp16 == 327_680
    assert accounting.kv_bytes(80, 1, 8, 128, 1) * 2 == fp16
    assert fp16 // accounting.kv_bytes(80, 1, 8, 128, 1) == 2
