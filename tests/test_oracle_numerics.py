"""Pins of oracle.numerics (bit decoding) and of the input rounding in workloads."""
import struct

import numpy as np
import torch

import workloads
from oracle.numerics import to_f64


def test_bits_decode_against_struct():
    rng = np.random.default_rng(0)
    b16 = rng.integers(0, 1 << 16, size=2000, dtype=np.uint16)
    b16 = b16[(b16 & 0x7C00) != 0x7C00]  # finite fp16 only
    f16 = to_f64(b16, "f16")
    for b, v in zip(b16.tolist(), f16.tolist()):
        assert struct.unpack("<e", struct.pack("<H", b))[0] == v
    bb = rng.integers(0, 1 << 16, size=2000, dtype=np.uint16)
    bb = bb[(bb & 0x7F80) != 0x7F80]  # finite bf16 only
    fb = to_f64(bb, "bf16")
    for b, v in zip(bb.tolist(), fb.tolist()):
        assert struct.unpack("<f", struct.pack("<I", b << 16))[0] == v
    x = rng.standard_normal(100).astype(np.float32)
    assert np.array_equal(to_f64(x, "f32"), x.astype(np.float64))


def test_input_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(1 << 16) * np.exp(rng.uniform(-20, 20, 1 << 16))).astype(np.float32)
    # include exact ties
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    got = workloads.round_to_dtype_bits(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    with np.errstate(over="ignore"):  # large magnitudes overflow to inf on both sides
        got = workloads.round_to_dtype_bits(x, "f16")
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_generator_rounding_path_matches_plain_rounding():
    # the chunked generator must give the same bits as rounding its own draws
    w = workloads.make_custom([40, 3], hq=2, hkv=1, d=8, dtype="bf16", seed=6)
    rng = np.random.Generator(np.random.PCG64(6))
    rng.permutation(w.num_blocks)
    q = rng.standard_normal(w.q.size, dtype=np.float32)
    assert np.array_equal(workloads.round_to_dtype_bits(q, "bf16").reshape(w.q.shape), w.q)
