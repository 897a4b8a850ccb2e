"""Reference decode attention over a paged KV cache (oracle; test infrastructure only).

One decode step computes, for every sequence and query head, the attention of
the single new query against the K and V of every token of the sequence so far,
which sit in the cache ("KV Cache for the intermediate", section "Precise
scientific definition": a new Q per new token, K and V of all earlier tokens
kept in memory for the attention dot product).  Under grouped-query attention a
group of query heads shares one K/V head (same page, section "Grouped Query
Attention (GQA)": 64 query heads over 8 KV heads for Llama 3 70B).  Paging moves
bytes, not results: the output equals attention over the sequence laid out
contiguously ("What PagedAttention is and what it changed in LLM serving",
sections "PagedAttention simply" and "FAQ").

Readings (the pages print no attention formula):
* textbook scaled dot-product attention, softmax over positions 0..len-1;
  the scale is an argument (the workloads use 1/sqrt(head_dim));
* query head h reads KV head h // (num_q_heads // num_kv_heads);
* the sequence length counts the token being decoded, whose K/V were written
  into the cache before attention; a sequence of length 0 gives zeros;
* splitting the positions into partitions and merging them with the running
  maximum / log-sum-exp rule (Milakov and Gimelshein, "Online normalizer
  calculation for softmax", 2018) gives the same result; ``partials`` and
  ``merge`` write that rule out for the tests of split-K.

``paged_prefill`` extends decode to a chunk of several new tokens per
sequence, each attending causally (pins in tests/test_oracle_prefill.py: one
token equals ``paged_decode`` bit for bit, a whole prompt equals torch's
causal scaled_dot_product_attention in float64, later positions cannot
change earlier outputs, brute force on tiny inputs).

Pins (tests/test_oracle_attention.py): brute force with Python scalars on tiny
inputs, torch's scaled_dot_product_attention in float64, invariance under any
relabelling of physical blocks, weights that sum to 1, len=1 -> v_0 exactly,
scale=0 -> mean of V, per-head constant V (pins the head grouping), a planted
"needle" key (pins the gather), MHA and MQA shapes, and split == unsplit.
"""
import numpy as np

from .numerics import to_f64

BLOCK_SIZE = 16


def gather(cache_bits, table_row, length: int, kv_head: int, dtype: str) -> np.ndarray:
    """Rows of positions 0..length-1 of one KV head, as float64 [length, D]."""
    pos = np.arange(int(length))
    blocks = np.asarray(table_row, dtype=np.int64)[pos // BLOCK_SIZE]
    return to_f64(cache_bits[blocks, kv_head, pos % BLOCK_SIZE, :], dtype)


def softmax_weights(q_h, K, scale: float) -> np.ndarray:
    """exp(scale*q.k_t - max) / sum over t."""
    x = scale * (K @ q_h)
    w = np.exp(x - x.max())
    return w / w.sum()


def attend(q_h, K, V, scale: float) -> np.ndarray:
    """Attention of one query vector over contiguous K, V (float64)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    return softmax_weights(q_h, K, scale) @ V


def paged_decode(q_bits, k_cache_bits, v_cache_bits, block_tables, context_lens,
                 scale: float, dtype: str) -> np.ndarray:
    """out[s, h] = attention(q[s, h], K_s, V_s), K_s/V_s gathered through the table.

    q_bits [S, Hq, D]; caches [NB, Hkv, 16, D] (logical view); block_tables
    [S, >=ceil(len/16)]; context_lens [S].  Returns float64 [S, Hq, D].
    """
    S, Hq, D = q_bits.shape
    Hkv = k_cache_bits.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // Hkv
    q = to_f64(q_bits, dtype)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        length = int(context_lens[s])
        if length == 0:
            continue
        for g in range(Hkv):
            K = gather(k_cache_bits, block_tables[s], length, g, dtype)
            V = gather(v_cache_bits, block_tables[s], length, g, dtype)
            for h in range(g * group, (g + 1) * group):
                out[s, h] = attend(q[s, h], K, V, scale)
    return out


def paged_prefill(q_bits, k_cache_bits, v_cache_bits, block_tables, query_start, context_lens,
                  scale: float, dtype: str) -> np.ndarray:
    """Attention of a chunk of new tokens per sequence (chunked prefill).

    Every token needs the K and V of all tokens before it ("KV Cache and
    PagedAttention: why your LLM server slows down", second article, section
    "What is the KV cache?"); a chunk of n_s new tokens of sequence s whose
    K/V are already in the cache (like the decoded token, reading R2) are the
    last n_s of its len_s positions, and query i of the chunk, at position
    p = len_s - n_s + i, attends to positions 0..p (causal).  n_s = 1 is
    decode.  q_bits [T, Hq, D] holds the chunks back to back: sequence s owns
    rows query_start[s] .. query_start[s+1]-1.  Returns float64 [T, Hq, D].
    """
    T, Hq, D = q_bits.shape
    Hkv = k_cache_bits.shape[1]
    group = Hq // Hkv
    q = to_f64(q_bits, dtype)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(len(context_lens)):
        a, b = int(query_start[s]), int(query_start[s + 1])
        length = int(context_lens[s])
        n = b - a
        if n == 0:
            continue
        if n > length:
            raise ValueError("a chunk cannot be longer than its sequence")
        for g in range(Hkv):
            K = gather(k_cache_bits, block_tables[s], length, g, dtype)
            V = gather(v_cache_bits, block_tables[s], length, g, dtype)
            for i in range(n):
                p = length - n + i
                for h in range(g * group, (g + 1) * group):
                    out[a + i, h] = attend(q[a + i, h], K[:p + 1], V[:p + 1], scale)
    return out


def partials(q_h, K, V, scale: float, partition_size: int):
    """Per partition of positions: (running max m, sum l, unnormalised acc)."""
    parts = []
    for a in range(0, K.shape[0], partition_size):
        x = scale * (K[a:a + partition_size] @ q_h)
        m = x.max()
        e = np.exp(x - m)
        parts.append((m, e.sum(), e @ V[a:a + partition_size]))
    return parts


def merge(parts) -> np.ndarray:
    """Combine partitions: M = max m_p; out = sum e^(m_p-M) acc_p / sum e^(m_p-M) l_p."""
    M = max(m for m, _, _ in parts)
    num = sum(np.exp(m - M) * acc for m, _, acc in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    return num / den
