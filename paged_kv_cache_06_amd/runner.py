"""Run a batch through the library: host tables from the C++ pool, then the kernels.

A batch description (duck-typed: the fields of ``workloads.Workload``) names the
sequences, their shared prompts, private tokens, the pool size and the pool's
initial order, and holds the token values.  The runner turns it into calls:

  A1  per sequence in index order: the first sequence of a prompt appends the
      prompt's tokens; later sequences of that prompt fork its table;
  A2  per sequence: append the private tokens before the step;
  B   per sequence: append the step's tokens (the last ``step_lens``).

Each phase becomes ``copy_blocks`` of its copy-on-write pairs followed by
``reshape_and_cache`` of its tokens; A1 and A2 are the prefill, B plus
``paged_attention_decode`` is the step.  Nothing here computes on values.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import (BLOCK_SIZE, PARTITION_AUTO, BlockManager, Pool, copy_blocks, decode_step,
               decode_step_int8, decode_step_int8_shared, decode_step_shared, new_kv_cache,
               new_kv_cache_int8, paged_attention_decode, paged_attention_decode_int8,
               paged_attention_decode_int8_shared, paged_attention_decode_shared,
               paged_attention_prefill, reshape_and_cache, reshape_and_cache_int8,
               shared_prefix_groups)

_TORCH_DTYPE = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}
NAN_FILL = float("nan")


def torch_dtype(dtype: str):
    import torch
    return getattr(torch, _TORCH_DTYPE[dtype])


def to_device(bits: np.ndarray, dtype: str, device="cuda"):
    """Storage bits (uint16 for bf16/fp16, float32) -> device tensor of ``dtype``."""
    import torch
    a = np.ascontiguousarray(bits)
    if dtype == "f32":
        t = torch.from_numpy(a)
    else:
        t = torch.from_numpy(a.view(np.int16)).view(torch_dtype(dtype))
    return t.to(device)


@dataclass
class HostPhase:
    pairs: np.ndarray  # int64 [n, 2]
    slots: np.ndarray  # int64 [T]
    key: np.ndarray  # bits [T, Hkv, D]
    value: np.ndarray


def plan(w, prefix_cache: bool = False):
    """Host side of the batch: (BlockManager, [A1, A2, B] phases).  With
    ``prefix_cache`` the sequences of a shared prompt take its whole blocks
    from the pool's prefix cache instead of forking the first one."""
    s_count = w.num_seqs
    lens = np.asarray(w.context_lens, dtype=np.int64)
    max_blocks = max(1, int(-(-lens.max() // BLOCK_SIZE)))
    pool = Pool(w.num_blocks, w.free_order)
    bm = BlockManager(pool, s_count, max_blocks, pad=w.num_blocks)
    poff = np.asarray(w.prompt_offsets)
    voff = np.asarray(w.private_offsets)
    hkv, d = w.num_kv_heads, w.head_dim

    def phase(pairs, slots, ks, vs):
        if ks:
            key, value = np.concatenate(ks), np.concatenate(vs)
        else:
            key = np.zeros((0, hkv, d), dtype=w.q.dtype)
            value = key
        sl = np.concatenate(slots) if slots else np.zeros(0, np.int64)
        return HostPhase(np.asarray(pairs, np.int64).reshape(-1, 2), sl.astype(np.int64), key,
                         value)

    # A1
    owner = {}
    slots, ks, vs = [], [], []
    for s in range(s_count):
        p = int(w.prompt_of[s])
        if p < 0:
            continue
        if prefix_cache:
            toks = w.prompt_tokens(p)
            i0 = bm.match(s, toks)
            sl, cow = bm.append(s, len(toks) - i0)
            assert cow is None
            slots.append(sl)
            ks.append(w.k_prompt[poff[p] + i0:poff[p + 1]])
            vs.append(w.v_prompt[poff[p] + i0:poff[p + 1]])
            bm.register(s, toks)
            continue
        if p in owner:
            bm.fork(s, owner[p])
            continue
        owner[p] = s
        sl, cow = bm.append(s, int(w.prompt_lens[p]))
        assert cow is None
        slots.append(sl)
        ks.append(w.k_prompt[poff[p]:poff[p + 1]])
        vs.append(w.v_prompt[poff[p]:poff[p + 1]])
    phases = [phase([], slots, ks, vs)]

    # A2 then B
    for which in ("history", "step"):
        pairs, slots, ks, vs = [], [], [], []
        for s in range(s_count):
            priv, step = int(w.private_lens[s]), int(w.step_lens[s])
            i0, n = (0, priv - step) if which == "history" else (priv - step, step)
            if n == 0:
                continue
            sl, cow = bm.append(s, n)
            if cow is not None:
                pairs.append(cow)
            slots.append(sl)
            a = int(voff[s]) + i0
            ks.append(w.k_private[a:a + n])
            vs.append(w.v_private[a:a + n])
        phases.append(phase(pairs, slots, ks, vs))
    return bm, phases


class DeviceBatch:
    """Device tensors of one batch and the calls of its prefill and step.

    The caches hold ``num_blocks + 1`` blocks: the extra block (id
    ``num_blocks``) is filled with NaN and every unused table entry points at
    it, as do all never-written slots, so any read past a sequence's end
    shows up in the output.  ``copies`` > 1 keeps that many independent caches
    (same tables) for benchmarks that must not hit in the last-level cache.
    ``int8`` keeps an INT8 cache with the workload's per-channel scales (its
    poison block and unwritten slots hold code 127).  ``shared_prefix``
    decodes through the shared-prefix calls, with the groups of sequences
    whose tables begin with the same blocks after the step.
    """

    def __init__(self, w, device="cuda", copies: int = 1, fill: float | None = NAN_FILL,
                 prefix_cache: bool = False, int8: bool = False, shared_prefix: bool = False):
        import torch

        self.w = w
        self.device = device
        self.torch_dtype = torch_dtype(w.dtype)
        self.bm, self.phases = plan(w, prefix_cache)
        self.num_blocks = w.num_blocks + 1  # + poison block
        self.tables = torch.from_numpy(self.bm.rows.copy()).to(device)
        self.context_lens = torch.from_numpy(np.asarray(w.context_lens, np.int32)).to(device)
        self.max_context_len = int(np.max(w.context_lens))
        self.int8 = int8
        if int8:  # INT8 cache: the poison and unwritten slots hold code 127
            sk, sv = w.int8_scales()
            self.k_scale = torch.from_numpy(sk).to(device)
            self.v_scale = torch.from_numpy(sv).to(device)
            self.caches = [new_kv_cache_int8(self.num_blocks, w.num_kv_heads, w.head_dim, device,
                                             None if fill is None else 127)
                           for _ in range(copies)]
        else:
            self.caches = [new_kv_cache(self.num_blocks, w.num_kv_heads, w.head_dim,
                                        self.torch_dtype, device, fill) for _ in range(copies)]
        self.q = self._dev(w.q)
        self.out = torch.empty(w.q.shape, dtype=self.torch_dtype, device=device)
        self.dev_phases = [self._dev_phase(ph) for ph in self.phases]
        self.shared = None
        if shared_prefix:
            seqs, start, blocks = shared_prefix_groups(self.bm.rows, self.bm.nblocks)
            self.shared = tuple(torch.from_numpy(x).to(device) for x in (seqs, start, blocks))

    def _dev(self, bits):
        return to_device(bits, self.w.dtype, self.device)

    def _dev_phase(self, ph: HostPhase):
        import torch

        return {"pairs": torch.from_numpy(ph.pairs).to(self.device),
                "slots": torch.from_numpy(ph.slots).to(self.device),
                "key": self._dev(ph.key), "value": self._dev(ph.value)}

    def _apply(self, ph, cache):
        kc, vc = cache
        if ph["pairs"].shape[0]:
            copy_blocks(kc, vc, ph["pairs"])
        if ph["slots"].shape[0]:
            if self.int8:
                reshape_and_cache_int8(ph["key"], ph["value"], kc, vc, ph["slots"], self.k_scale,
                                       self.v_scale)
            else:
                reshape_and_cache(ph["key"], ph["value"], kc, vc, ph["slots"])

    def prefill(self):
        for cache in self.caches:
            for ph in self.dev_phases[:2]:
                self._apply(ph, cache)

    def step(self, copy: int = 0, partition_size: int = PARTITION_AUTO, out=None,
             fused: bool = True):
        """The step: block copies (if any), then the new tokens' cache writes and
        the decode -- through decode_step / decode_step_int8 (one launch fewer)
        unless ``fused`` is False."""
        cache = self.caches[copy]
        ph = self.dev_phases[2]
        if not fused or ph["slots"].shape[0] == 0:
            self._apply(ph, cache)
            self.decode(copy, partition_size, out)
            return
        kc, vc = cache
        if ph["pairs"].shape[0]:
            copy_blocks(kc, vc, ph["pairs"])
        o = self.out if out is None else out
        if self.int8 and self.shared is not None:
            decode_step_int8_shared(ph["key"], ph["value"], ph["slots"], self.q, kc, vc,
                                    self.k_scale, self.v_scale, self.tables, self.context_lens,
                                    *self.shared, self.w.scale, o,
                                    max_context_len=self.max_context_len,
                                    partition_size=partition_size)
            return
        if self.int8:
            decode_step_int8(ph["key"], ph["value"], ph["slots"], self.q, kc, vc, self.k_scale,
                             self.v_scale, self.tables, self.context_lens, self.w.scale, o,
                             max_context_len=self.max_context_len, partition_size=partition_size)
            return
        if self.shared is not None:
            decode_step_shared(ph["key"], ph["value"], ph["slots"], self.q, kc, vc, self.tables,
                               self.context_lens, *self.shared, self.w.scale, o,
                               max_context_len=self.max_context_len,
                               partition_size=partition_size)
            return
        decode_step(ph["key"], ph["value"], ph["slots"], self.q, kc, vc, self.tables,
                    self.context_lens, self.w.scale, o, max_context_len=self.max_context_len,
                    partition_size=partition_size)

    def decode(self, copy: int = 0, partition_size: int = PARTITION_AUTO, out=None):
        kc, vc = self.caches[copy]
        if self.int8 and self.shared is not None:
            paged_attention_decode_int8_shared(self.q, kc, vc, self.k_scale, self.v_scale,
                                               self.tables, self.context_lens, *self.shared,
                                               self.w.scale, self.out if out is None else out,
                                               max_context_len=self.max_context_len,
                                               partition_size=partition_size)
            return
        if self.int8:
            paged_attention_decode_int8(self.q, kc, vc, self.k_scale, self.v_scale, self.tables,
                                        self.context_lens, self.w.scale,
                                        self.out if out is None else out,
                                        max_context_len=self.max_context_len,
                                        partition_size=partition_size)
            return
        if self.shared is not None:
            paged_attention_decode_shared(self.q, kc, vc, self.tables, self.context_lens,
                                          *self.shared, self.w.scale,
                                          self.out if out is None else out,
                                          max_context_len=self.max_context_len,
                                          partition_size=partition_size)
            return
        paged_attention_decode(self.q, kc, vc, self.tables, self.context_lens, self.w.scale,
                               self.out if out is None else out,
                               max_context_len=self.max_context_len,
                               partition_size=partition_size)

    def attend_chunks(self, copy: int = 0, out=None):
        """Chunked prefill of a batch with ``chunk_q``: the step's tokens
        (phase B, already written) attend causally; returns the output tensor."""
        import torch
        if not hasattr(self, "chunk_q"):
            self.chunk_q = self._dev(self.w.chunk_q)
            self.query_start = torch.from_numpy(self.w.query_start).to(self.device)
            self.chunk_out = torch.empty_like(self.chunk_q)
            self.max_chunk = int(np.max(self.w.step_lens))
        kc, vc = self.caches[copy]
        o = self.chunk_out if out is None else out
        paged_attention_prefill(self.chunk_q, kc, vc, self.tables, self.query_start,
                                self.context_lens, self.w.scale, o, max_chunk_len=self.max_chunk)
        return o

    def out_bits(self, out=None) -> np.ndarray:
        import torch

        o = (self.out if out is None else out).cpu()
        if self.w.dtype != "f32":
            return o.view(torch.int16).numpy().view(np.uint16)
        return o.numpy()
