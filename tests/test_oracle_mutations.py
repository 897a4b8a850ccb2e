"""Planted mistakes in the oracle (CPU only): each must make one of its pins fail.

A pin that passes whatever the oracle does pins nothing; these tests patch a
plausible mistake into one oracle step and check that the pin covering that
step catches it.
"""
import numpy as np
import pytest

from oracle import attention, pool
from tests import test_oracle_attention as ta
from tests import test_oracle_pool as tp

_orig_gather = attention.gather


def _wrong_head(cache, table_row, length, kv_head, dtype):
    return _orig_gather(cache, table_row, length, (kv_head + 1) % cache.shape[1], dtype)


def _wrong_row(cache, table_row, length, kv_head, dtype):
    pos = np.arange(int(length))
    blocks = np.asarray(table_row, dtype=np.int64)[pos // 16]
    return attention.to_f64(cache[blocks, kv_head, (pos + 1) % 16, :], dtype)


def _wrong_sign(q_h, K, scale):
    x = -scale * (K @ q_h)
    w = np.exp(x - x.max())
    return w / w.sum()


def _transposed(q_h, K, scale):
    x = scale * (K[:, ::-1] @ q_h)  # operand read along the wrong axis order
    w = np.exp(x - x.max())
    return w / w.sum()


def _merge_drops_rescale(parts):
    M = max(m for m, _, _ in parts)
    num = sum(np.exp(m - M) * acc for m, _, acc in parts)
    den = sum(l for _, l, _ in parts)
    return num / den


@pytest.mark.parametrize("target,name,bad,pin", [
    (attention, "gather", _wrong_head,
     lambda: ta.test_paged_decode_equals_brute_force_on_contiguous_sequences("f32")),
    (attention, "gather", _wrong_head, ta.test_constant_values_per_kv_head_pin_the_grouping),
    (attention, "gather", _wrong_row, ta.test_needle_key_pins_the_gather),
    (attention, "gather", _wrong_row, ta.test_paged_decode_matches_torch_sdpa_float64),
    (attention, "softmax_weights", _wrong_sign,
     lambda: ta.test_paged_decode_equals_brute_force_on_contiguous_sequences("bf16")),
    (attention, "softmax_weights", _transposed, ta.test_paged_decode_matches_torch_sdpa_float64),
    (attention, "merge", _merge_drops_rescale, lambda: ta.test_split_merge_equals_unsplit(512)),
], ids=["head", "head-const", "row-needle", "row-sdpa", "sign", "transpose", "merge"])
def test_planted_attention_mistake_is_caught(monkeypatch, target, name, bad, pin):
    monkeypatch.setattr(target, name, bad)
    with pytest.raises(AssertionError):
        pin()


def test_planted_fifo_reuse_is_caught(monkeypatch):
    def fifo_free(self, b):
        b = self._check(b)
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free_stack.insert(0, b)  # bottom of the stack: handed out last
    monkeypatch.setattr(pool.BlockPool, "free", fifo_free)
    with pytest.raises(AssertionError):
        tp.test_free_order_and_lifo_reuse()


def test_planted_cow_without_release_is_caught(monkeypatch):
    orig = pool.BlockPool.free
    calls = {"n": 0}

    def leaky_free(self, b):
        # forget to drop the source's reference during copy-on-write
        import inspect
        if inspect.stack()[1].function == "append":
            calls["n"] += 1
            return
        orig(self, b)
    monkeypatch.setattr(pool.BlockPool, "free", leaky_free)
    with pytest.raises(AssertionError):
        tp.test_copy_on_write_first_writers_copy_last_writes_in_place()
    assert calls["n"] > 0


from tests import test_oracle_prefix as tpre  # noqa: E402


def test_planted_block_id_keys_are_caught(monkeypatch):
    """Keying a cached block on its parent's block id (reused after eviction)
    instead of a never-reused serial number gives false hits."""
    monkeypatch.setattr(pool.BlockPool, "_chain_id", lambda self, b: b + 1)
    with pytest.raises(AssertionError):
        tpre.test_no_false_hit_through_a_reused_block_id()


def test_planted_mru_eviction_is_caught(monkeypatch):
    orig_alloc = pool.BlockPool.alloc

    def mru_alloc(self):
        if not self.free_stack and self.lru:
            self.lru.reverse()
            try:
                return orig_alloc(self)
            finally:
                self.lru.reverse()
        return orig_alloc(self)
    monkeypatch.setattr(pool.BlockPool, "alloc", mru_alloc)
    with pytest.raises(AssertionError):
        tpre.test_uncached_blocks_go_first_then_least_recently_released()


def test_planted_match_without_reference_is_caught(monkeypatch):
    orig_match = pool.BlockPool.match_prefix

    def match_no_ref(self, tokens):
        found = orig_match(self, tokens)
        for b in found:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.lru.append(b)
        return found
    monkeypatch.setattr(pool.BlockPool, "match_prefix", match_no_ref)
    with pytest.raises((AssertionError, pool.PoolError)):  # a count check, or a later call on an unheld block
        tpre.test_cached_blocks_outlive_their_sequence()


from oracle import quant  # noqa: E402
from tests import test_oracle_quant as tq  # noqa: E402


def _quantize_with(rounding, lo=-127):
    def q(bits, dtype, scale):
        from oracle.numerics import to_f64
        x = to_f64(bits, dtype).astype(np.float32)
        with np.errstate(over="ignore", invalid="ignore"):
            y = rounding(x / np.asarray(scale, np.float32))
        y = np.where(np.isnan(y), np.float32(0), y)
        return np.clip(y, lo, 127).astype(np.int8)
    return q


@pytest.mark.parametrize("bad,pin", [
    (_quantize_with(np.trunc), lambda: tq.test_codes_are_the_nearest_integer_of_the_exact_ratio("bf16")),
    (_quantize_with(lambda y: np.sign(y) * np.floor(np.abs(y) + 0.5)),
     tq.test_ties_go_to_even_and_sign_is_symmetric),
    (_quantize_with(np.rint, lo=-128), tq.test_saturation_infinities_nan_and_no_minus_128),
], ids=["truncate", "half-away", "minus-128"])
def test_planted_quantization_mistake_is_caught(monkeypatch, bad, pin):
    monkeypatch.setattr(quant, "quantize", bad)
    with pytest.raises(AssertionError):
        pin()


from oracle import cache_ops  # noqa: E402
from tests import test_oracle_swap as tsw  # noqa: E402


def test_planted_swap_without_release_is_caught(monkeypatch):
    def leaky(src, dst, blocks):
        blocks = [src._check(b) for b in blocks]
        if dst.num_free() < len(blocks):
            raise pool.OutOfBlocks("short")
        return [(b, dst.alloc()) for b in blocks]  # forgets to release the source
    monkeypatch.setattr(pool, "swap_blocks", leaky)
    monkeypatch.setattr(tsw, "swap_blocks", leaky)
    with pytest.raises(AssertionError):
        tsw.test_random_swaps_conserve_references_in_both_tiers()


def test_planted_per_listing_check_is_caught(monkeypatch):
    def per_listing(src, dst, blocks):
        if dst.num_free() < len(blocks):
            raise pool.OutOfBlocks("short")
        pairs = []
        for b in blocks:  # checks each listing as it comes, after earlier frees
            src._check(b)
            pairs.append((int(b), dst.alloc()))
            src.free(b)
        return pairs
    monkeypatch.setattr(tsw, "swap_blocks", per_listing)
    with pytest.raises(AssertionError):
        tsw.test_a_block_listed_more_often_than_held_changes_nothing()


def test_planted_backwards_transfer_is_caught(monkeypatch):
    def backwards(src_k, src_v, dst_k, dst_v, pairs):
        for s, d in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
            dst_k[s] = src_k[d]
            dst_v[s] = src_v[d]
    monkeypatch.setattr(cache_ops, "transfer_blocks", backwards)
    with pytest.raises((AssertionError, IndexError)):
        tsw.test_swap_out_and_back_in_restores_every_sequence_exactly()


from tests import test_oracle_prefill as tpf  # noqa: E402


def _prefill_window(extra):
    def bad(q_bits, k_cache_bits, v_cache_bits, block_tables, query_start, context_lens, scale,
            dtype):
        T, Hq, D = q_bits.shape
        group = Hq // k_cache_bits.shape[1]
        q = attention.to_f64(q_bits, dtype)
        out = np.zeros((T, Hq, D))
        for s in range(len(context_lens)):
            a, b = int(query_start[s]), int(query_start[s + 1])
            length, n = int(context_lens[s]), b - a
            for g in range(k_cache_bits.shape[1]):
                K = attention.gather(k_cache_bits, block_tables[s], length, g, dtype)
                V = attention.gather(v_cache_bits, block_tables[s], length, g, dtype)
                for i in range(n):
                    p = length if extra is None else length - n + i + extra
                    for h in range(g * group, (g + 1) * group):
                        out[a + i, h] = attention.attend(q[a + i, h], K[:p], V[:p], scale)
        return out
    return bad


@pytest.mark.parametrize("bad,pin", [
    (_prefill_window(0), tpf.test_one_token_chunks_are_decode_bit_for_bit),  # drops position p
    (_prefill_window(None), tpf.test_later_positions_cannot_change_earlier_queries),  # not causal
    (_prefill_window(None), tpf.test_whole_prompts_match_torch_causal_sdpa_float64),
], ids=["off-by-one", "non-causal", "non-causal-sdpa"])
def test_planted_prefill_mistake_is_caught(monkeypatch, bad, pin):
    monkeypatch.setattr(attention, "paged_prefill", bad)
    with pytest.raises(AssertionError):
        pin()
