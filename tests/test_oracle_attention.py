"""Pins of oracle.attention (and the cache/table path of oracle.step feeding it)."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, step
from oracle.numerics import to_f64

NAN_BITS = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}


def _brute_force(q, K, V, scale):
    """Python scalars only: no numpy products, no vector softmax."""
    L, D = len(K), len(q)
    scores = [scale * sum(q[i] * K[t][i] for i in range(D)) for t in range(L)]
    m = max(scores)
    e = [math.exp(x - m) for x in scores]
    tot = sum(e)
    return [sum(e[t] * V[t][i] for t in range(L)) / tot for i in range(D)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_paged_decode_equals_brute_force_on_contiguous_sequences(dtype):
    w = workloads.make_custom([1, 5, 16, 17, 40], hq=4, hkv=2, d=8, dtype=dtype, seed=11)
    pl, kc, vc, out = step.run(w, NAN_BITS[dtype])
    group = w.num_q_heads // w.num_kv_heads
    q = to_f64(w.q, dtype)
    for s in range(w.num_seqs):
        kb, vb = w.sequence_kv(s)  # generator order, never through a table
        K, V = to_f64(kb, dtype), to_f64(vb, dtype)
        for h in range(w.num_q_heads):
            g = h // group
            ref = _brute_force(q[s, h].tolist(), K[:, g].tolist(), V[:, g].tolist(), w.scale)
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-12, atol=1e-14)


def test_paged_decode_matches_torch_sdpa_float64():
    w = workloads.make_custom([3, 64, 100, 257], hq=8, hkv=2, d=32, dtype="bf16", seed=5)
    pl, kc, vc, out = step.run(w, NAN_BITS["bf16"])
    group = w.num_q_heads // w.num_kv_heads
    q = torch.from_numpy(to_f64(w.q, "bf16"))
    for s in range(w.num_seqs):
        kb, vb = w.sequence_kv(s)
        K = torch.from_numpy(to_f64(kb, "bf16")).permute(1, 0, 2)  # [Hkv, L, D]
        V = torch.from_numpy(to_f64(vb, "bf16")).permute(1, 0, 2)
        K = K.repeat_interleave(group, dim=0).unsqueeze(0)
        V = V.repeat_interleave(group, dim=0).unsqueeze(0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[s].unsqueeze(0).unsqueeze(2), K, V, scale=w.scale)[0, :, 0]
        np.testing.assert_allclose(out[s], ref.numpy(), rtol=1e-11, atol=1e-13)


def test_block_relabelling_leaves_output_bit_identical():
    w = workloads.make_custom([7, 33, 48, 90], hq=4, hkv=2, d=16, dtype="bf16", seed=3)
    pl, kc, vc, out = step.run(w, NAN_BITS["bf16"])
    perm = np.random.default_rng(0).permutation(w.num_blocks)  # new id of old block b
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    width = max(len(t) for t in pl.tables)
    tables = pl.padded_tables(width, 0)
    out2 = attention.paged_decode(w.q, kc2, vc2, perm[tables], pl.context_lens, w.scale, "bf16")
    assert np.array_equal(out, out2)


def test_weights_sum_to_one_and_special_cases():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(16)
    K = rng.standard_normal((50, 16))
    V = rng.standard_normal((50, 16))
    w = attention.softmax_weights(q, K, 0.3)
    assert abs(w.sum() - 1.0) < 1e-12 and np.all(w > 0)
    # one position: the output is that position's value, exactly
    assert np.array_equal(attention.attend(q, K[:1], V[:1], 0.3), V[0])
    # zero scale: uniform weights, the mean of V
    np.testing.assert_allclose(attention.attend(q, K, V, 0.0), V.mean(axis=0), rtol=1e-13)
    # no positions: zeros
    assert np.array_equal(attention.attend(q, K[:0], V[:0], 0.3), np.zeros(16))


def test_constant_values_per_kv_head_pin_the_grouping():
    w = workloads.make_custom([20, 35], hq=8, hkv=4, d=8, dtype="f32", seed=2)
    pl, kc, vc, _ = step.run(w, NAN_BITS["f32"])
    for g in range(4):
        vc[:, g] = np.float32(g)
    width = max(len(t) for t in pl.tables)
    out = attention.paged_decode(w.q, kc, vc, pl.padded_tables(width, 0), pl.context_lens,
                                 w.scale, "f32")
    for h in range(8):
        np.testing.assert_allclose(out[:, h], h // 2, rtol=1e-14, atol=0)


def test_needle_key_pins_the_gather():
    w = workloads.make_custom([45], hq=2, hkv=1, d=16, dtype="f32", seed=9)
    pl, kc, vc, _ = step.run(w, NAN_BITS["f32"])
    table = pl.tables[0]
    width = len(table)
    q = to_f64(w.q, "f32")
    for j in (0, 15, 16, 31, 44):
        kc2 = kc.copy()
        blk, row = table[j // 16], j % 16
        kc2[blk, 0, row] = (50.0 * q[0, 0]).astype(np.float32)
        out = attention.paged_decode(w.q, kc2, vc, pl.padded_tables(width, 0),
                                     pl.context_lens, 1.0, "f32")
        np.testing.assert_allclose(out[0, 0], vc[blk, 0, row].astype(np.float64), atol=1e-9)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 1)])
def test_mha_and_mqa_shapes(hq, hkv):
    w = workloads.make_custom([9, 30], hq=hq, hkv=hkv, d=8, dtype="f16", seed=4)
    _, _, _, out = step.run(w, NAN_BITS["f16"])
    q = to_f64(w.q, "f16")
    for s in range(2):
        kb, vb = w.sequence_kv(s)
        K, V = to_f64(kb, "f16"), to_f64(vb, "f16")
        for h in range(hq):
            g = h // (hq // hkv)
            ref = _brute_force(q[s, h].tolist(), K[:, g].tolist(), V[:, g].tolist(), w.scale)
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-12)


def test_zero_length_sequence_gives_zeros():
    w = workloads.make_custom([5, 9], hq=2, hkv=1, d=8, dtype="f32", seed=1)
    pl, kc, vc, _ = step.run(w, NAN_BITS["f32"])
    out = attention.paged_decode(w.q, kc, vc, pl.padded_tables(1, 0), np.array([0, 0]),
                                 w.scale, "f32")
    assert np.array_equal(out, np.zeros_like(out))


@pytest.mark.parametrize("size", [1, 7, 16, 512])
def test_split_merge_equals_unsplit(size):
    rng = np.random.default_rng(size)
    q = rng.standard_normal(64)
    K = rng.standard_normal((1500, 64)) * 2
    V = rng.standard_normal((1500, 64))
    ref = attention.attend(q, K, V, 0.125)
    got = attention.merge(attention.partials(q, K, V, 0.125, size))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_shared_prefix_sequences_see_their_own_private_tokens():
    # 2 prompts x 3 samples; the step is where they diverge (copy-on-write)
    w = workloads.make_custom([1, 5, 20, 2, 3, 40], hq=4, hkv=2, d=8, dtype="bf16", seed=8,
                              prompt_lens=[21, 32], prompt_of=[0, 0, 0, 1, 1, 1])
    pl, kc, vc, out = step.run(w, NAN_BITS["bf16"])
    assert len(pl.phases[2].pairs) == 2  # prompt 0 has a partial block; prompt 1 does not
    q = to_f64(w.q, "bf16")
    for s in range(w.num_seqs):
        kb, vb = w.sequence_kv(s)
        K, V = to_f64(kb, "bf16"), to_f64(vb, "bf16")
        for h in range(4):
            ref = _brute_force(q[s, h].tolist(), K[:, h // 2].tolist(), V[:, h // 2].tolist(),
                               w.scale)
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-12)
