"""Reference run of one workload: allocate, write, copy, attend (oracle; tests only).

Order of a batch (the reading taken of the pages' serving story):

  A1  for each sequence in index order: the first sequence of a shared prompt
      allocates and writes the prompt; every later sequence of that prompt
      forks the first one's table (one more reference on every block);
  A2  for each sequence in index order: append its private tokens except the
      last ``step_len`` ones;
  B   (the step) for each sequence in index order: append its last ``step_len``
      tokens.

Each phase yields its copy-on-write pairs and the slots of the tokens it
appends; its effect on the cache is "copy the pairs, then write the tokens".
Then every sequence decodes its last token over all ``len`` cached positions.

With ``prefix_cache=True``, A1 runs through the pool's prefix cache instead of
forking: every sequence of a prompt looks the prompt's token ids up, takes the
cached whole blocks, allocates and writes the rest itself, and enters its full
blocks in the cache ("PagedAttention for the professional", serve-command
section on prefix caching).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import attention, cache_ops, quant
from .pool import BLOCK_SIZE as pool_block
from .pool import BlockPool


@dataclass
class Phase:
    pairs: np.ndarray  # int64 [n, 2] (src, dst)
    slots: np.ndarray  # int64 [T]
    key: np.ndarray  # bits [T, Hkv, D]
    value: np.ndarray


@dataclass
class Plan:
    pool: BlockPool
    tables: list  # per sequence: list of physical block ids
    phases: list  # [A1, A2, B]
    context_lens: np.ndarray

    def padded_tables(self, width: int, pad: int) -> np.ndarray:
        out = np.full((len(self.tables), width), pad, dtype=np.int32)
        for s, t in enumerate(self.tables):
            out[s, :len(t)] = t
        return out


def _phase(pairs, slots, keys, values, hkv, d, bits):
    if keys:
        k = np.concatenate(keys)
        v = np.concatenate(values)
    else:
        k = np.zeros((0, hkv, d), dtype=bits)
        v = np.zeros((0, hkv, d), dtype=bits)
    return Phase(np.asarray(pairs, dtype=np.int64).reshape(-1, 2),
                 np.asarray(slots, dtype=np.int64), k, v)


def plan(w, prefix_cache: bool = False) -> Plan:
    pool = BlockPool(w.num_blocks, w.free_order)
    S, hkv, d = w.num_seqs, w.num_kv_heads, w.head_dim
    bits = w.q.dtype
    tables = [[] for _ in range(S)]
    poff, voff = w.prompt_offsets, w.private_offsets

    # A1: prompts, then forks
    owner = {}
    pairs, slots, ks, vs = [], [], [], []
    for s in range(S):
        p = int(w.prompt_of[s])
        if p < 0:
            continue
        if prefix_cache:
            toks = w.prompt_tokens(p)
            tables[s] = pool.match_prefix(toks)
            i0 = len(tables[s]) * pool_block
            sl, cow = pool.append(tables[s], i0, len(toks) - i0)
            assert cow is None
            slots += sl
            ks.append(w.k_prompt[poff[p] + i0:poff[p + 1]])
            vs.append(w.v_prompt[poff[p] + i0:poff[p + 1]])
            pool.register(tables[s], toks)
        elif p not in owner:
            owner[p] = s
            n = int(w.prompt_lens[p])
            sl, cow = pool.append(tables[s], 0, n)
            assert cow is None
            slots += sl
            ks.append(w.k_prompt[poff[p]:poff[p + 1]])
            vs.append(w.v_prompt[poff[p]:poff[p + 1]])
        else:
            tables[s] = pool.fork(tables[owner[p]])
    phases = [_phase(pairs, slots, ks, vs, hkv, d, bits)]

    def start_of(s):
        p = int(w.prompt_of[s])
        return int(w.prompt_lens[p]) if p >= 0 else 0

    # A2: private history; B: the step
    for first, count in ((lambda s: 0, lambda s: int(w.private_lens[s] - w.step_lens[s])),
                         (lambda s: int(w.private_lens[s] - w.step_lens[s]),
                          lambda s: int(w.step_lens[s]))):
        pairs, slots, ks, vs = [], [], [], []
        for s in range(S):
            i0, n = first(s), count(s)
            if n == 0:
                continue
            sl, cow = pool.append(tables[s], start_of(s) + i0, n)
            if cow is not None:
                pairs.append(cow)
            slots += sl
            a = voff[s] + i0
            ks.append(w.k_private[a:a + n])
            vs.append(w.v_private[a:a + n])
        phases.append(_phase(pairs, slots, ks, vs, hkv, d, bits))
    return Plan(pool, tables, phases, w.context_lens.copy())


def empty_cache(w, fill_bits) -> tuple:
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    k = np.full(shape, fill_bits, dtype=w.q.dtype)
    return k, k.copy()


def apply_phase(phase: Phase, k_cache, v_cache) -> None:
    cache_ops.copy_blocks(k_cache, v_cache, phase.pairs)
    cache_ops.reshape_and_cache(phase.key, phase.value, k_cache, v_cache, phase.slots)


def run(w, fill_bits, phases=None, prefix_cache: bool = False):
    """Plan, build the cache and decode.  Returns (plan, k_cache, v_cache, out)."""
    pl = plan(w, prefix_cache)
    k_cache, v_cache = empty_cache(w, fill_bits)
    for ph in (pl.phases if phases is None else [pl.phases[i] for i in phases]):
        apply_phase(ph, k_cache, v_cache)
    width = max(1, max(len(t) for t in pl.tables))
    out = attention.paged_decode(w.q, k_cache, v_cache, pl.padded_tables(width, 0),
                                 pl.context_lens, w.scale, w.dtype)
    return pl, k_cache, v_cache, out


def run_prefill(w, fill_bits):
    """``run`` for a chunked-prefill batch: after the step wrote every chunk's
    K/V, each chunk's queries (``w.chunk_q``) attend causally.  Returns (plan,
    k_cache, v_cache, out [T, Hq, D])."""
    pl = plan(w)
    k_cache, v_cache = empty_cache(w, fill_bits)
    for ph in pl.phases:
        apply_phase(ph, k_cache, v_cache)
    width = max(1, max(len(t) for t in pl.tables))
    out = attention.paged_prefill(w.chunk_q, k_cache, v_cache, pl.padded_tables(width, 0),
                                  w.query_start, pl.context_lens, w.scale, w.dtype)
    return pl, k_cache, v_cache, out


def run_int8(w, fill_code: int = 127, prefix_cache: bool = False):
    """``run`` over an INT8 cache with the workload's per-channel scales: the
    phases' tokens are quantized as they are written.  Returns (plan, k_codes,
    v_codes, out)."""
    pl = plan(w, prefix_cache)
    sk, sv = w.int8_scales()
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    k_codes = np.full(shape, fill_code, dtype=np.int8)
    v_codes = k_codes.copy()
    for ph in pl.phases:
        cache_ops.copy_blocks(k_codes, v_codes, ph.pairs)
        quant.reshape_and_cache(ph.key, ph.value, w.dtype, k_codes, v_codes, ph.slots, sk, sv)
    width = max(1, max(len(t) for t in pl.tables))
    out = quant.paged_decode(w.q, k_codes, v_codes, sk, sv, pl.padded_tables(width, 0),
                             pl.context_lens, w.scale, w.dtype)
    return pl, k_codes, v_codes, out


def decode_sequences(w, k_cache, v_cache, tables, seqs) -> np.ndarray:
    """Oracle output of selected sequences only, float64 [len(seqs), Hq, D]."""
    out = []
    lens = w.context_lens
    for s in seqs:
        out.append(attention.paged_decode(
            w.q[s:s + 1], k_cache, v_cache, [tables[s]], lens[s:s + 1], w.scale, w.dtype)[0])
    return np.stack(out)
