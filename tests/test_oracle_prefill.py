"""Pins of oracle.attention.paged_prefill (chunked prefill, causal)."""
import numpy as np
import torch

import workloads
from oracle import attention, step
from oracle.numerics import to_f64
from tests.helpers import NAN_BITS


def test_one_token_chunks_are_decode_bit_for_bit():
    w = workloads.make_custom([1, 17, 40, 300], hq=8, hkv=2, d=32, dtype="bf16", seed=2)
    pl, kc, vc, dec = step.run(w, NAN_BITS["bf16"])
    width = max(len(t) for t in pl.tables)
    qs = np.arange(w.num_seqs + 1, dtype=np.int32)
    pre = attention.paged_prefill(w.q, kc, vc, pl.padded_tables(width, 0), qs, pl.context_lens,
                                  w.scale, "bf16")
    assert np.array_equal(pre, dec)


def test_whole_prompts_match_torch_causal_sdpa_float64():
    w = workloads.make_prefill([5, 33, 70], [0, 0, 0], hq=8, hkv=2, d=32, dtype="bf16", seed=3)
    pl, kc, vc, out = step.run_prefill(w, NAN_BITS["bf16"])
    group = w.num_q_heads // w.num_kv_heads
    q = to_f64(w.chunk_q, "bf16")
    qs = w.query_start
    for s in range(w.num_seqs):
        kb, vb = w.sequence_kv(s)
        K = torch.from_numpy(to_f64(kb, "bf16")).permute(1, 0, 2).repeat_interleave(group, 0)
        V = torch.from_numpy(to_f64(vb, "bf16")).permute(1, 0, 2).repeat_interleave(group, 0)
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]]).permute(1, 0, 2)  # [Hq, n, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0), is_causal=True, scale=w.scale)[0]
        np.testing.assert_allclose(out[qs[s]:qs[s + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=1e-11, atol=1e-13)


def test_later_positions_cannot_change_earlier_queries():
    w = workloads.make_prefill([24], [10], hq=4, hkv=2, d=16, dtype="bf16", seed=4)
    pl, kc, vc, out = step.run_prefill(w, NAN_BITS["bf16"])
    table = pl.padded_tables(len(pl.tables[0]), 0)
    # overwrite the K/V of position 20 (chunk query 10): queries 0..9 keep their outputs
    b, r = divmod(20, 16)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[table[0, b], :, r, :] ^= np.uint16(0x0040)  # top mantissa bit: finite, clearly different
    vc2[table[0, b], :, r, :] ^= np.uint16(0x0040)  # top mantissa bit: finite, clearly different
    out2 = attention.paged_prefill(w.chunk_q, kc2, vc2, table, w.query_start, pl.context_lens,
                                   w.scale, "bf16")
    assert np.array_equal(out2[:10], out[:10])
    assert not np.allclose(out2[10:], out[10:])


def test_brute_force_tiny():
    w = workloads.make_prefill([3, 2], [2, 0], hq=2, hkv=1, d=4, dtype="bf16", seed=5)
    pl, kc, vc, out = step.run_prefill(w, NAN_BITS["bf16"])
    q = to_f64(w.chunk_q, "bf16")
    qs = w.query_start
    for s in range(2):
        kb, vb = w.sequence_kv(s)
        K, V = to_f64(kb, "bf16")[:, 0], to_f64(vb, "bf16")[:, 0]
        n, L = qs[s + 1] - qs[s], int(w.context_lens[s])
        for i in range(n):
            p = L - n + i
            for h in range(2):
                xs = [w.scale * sum(float(q[qs[s] + i, h, d]) * float(K[t, d]) for d in range(4))
                      for t in range(p + 1)]
                m = max(xs)
                e = [np.exp(x - m) for x in xs]
                want = [sum(e[t] * float(V[t, d]) for t in range(p + 1)) / sum(e) for d in range(4)]
                np.testing.assert_allclose(out[qs[s] + i, h], want, rtol=1e-12, atol=1e-14)
