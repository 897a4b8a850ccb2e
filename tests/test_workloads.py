"""Shape and distribution checks of the seeded workloads (structure only: fast)."""
import math

import numpy as np
import pytest

import workloads


def test_tiny_workload_is_as_specified():
    w = workloads.make(1)
    assert list(w.context_lens) == [1, 17, 33, 100]
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype) == (4, 2, 64, "f32")
    assert w.num_blocks == 64 and sorted(w.free_order) == list(range(64))
    assert w.scale == pytest.approx(1 / 8)
    assert w.q.shape == (4, 4, 64) and w.k_private.shape == (151, 2, 64)


def test_llama3_8b_lengths_uniform_in_range():
    w = workloads.make(2, values=False)
    lens = w.context_lens
    assert lens.shape == (64,) and lens.min() >= 128 and lens.max() <= 4096
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype) == (32, 8, 128, "bf16")
    need = int(np.sum(-(-lens // 16)))
    assert w.num_blocks == math.ceil(1.1 * need)


def test_llama3_70b_lengths_lognormal_clipped():
    w = workloads.make(3, values=False)
    lens = w.context_lens
    assert lens.shape == (256,) and lens.min() >= 16 and lens.max() <= 8192
    assert 200 < np.median(lens) < 420
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim) == (64, 8, 128)


def test_shared_prefix_structure():
    w = workloads.make(4, values=False)
    assert w.num_seqs == 256 and len(w.prompt_lens) == 64
    assert np.all((w.prompt_lens > 2048) & (w.prompt_lens < 2048 + 16))
    assert np.all((w.private_lens >= 1) & (w.private_lens <= 300))
    assert np.array_equal(w.step_lens, w.private_lens)
    assert list(np.bincount(w.prompt_of)) == [4] * 64
    w2 = workloads.make("4b", values=False)
    assert len(w2.prompt_lens) == 1 and np.all(w2.prompt_of == 0)


def test_long_context_structure():
    w = workloads.make(5, values=False)
    assert np.all(w.context_lens == 32768) and w.num_blocks == 18023
    assert w.dtype == "f16" and w.notes["partition_size"] == 512


def test_values_are_deterministic_and_structure_independent_of_values():
    a = workloads.make(2, values=False)
    b = workloads.make_custom([3, 4], hq=2, hkv=1, d=4, dtype="f16", seed=2)
    c = workloads.make_custom([3, 4], hq=2, hkv=1, d=4, dtype="f16", seed=2)
    assert np.array_equal(b.k_private, c.k_private) and np.array_equal(b.q, c.q)
    a2 = workloads.make(2, values=False)
    assert np.array_equal(a.context_lens, a2.context_lens)
    assert np.array_equal(a.free_order, a2.free_order)
