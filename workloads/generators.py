"""Seeded input generators for the five decode workloads and for ad-hoc test cases.

Every workload is drawn from ``numpy.random.Generator(PCG64(seed))``; the seed of
a named workload is its number (1..5).  Draw order, fixed so that both sides see
the same bits:

  1. sequence structure: context lengths (or, for the shared-prefix workloads,
     the prompt tails t_p and the private lengths);
  2. the initial free-list order of the block pool (a permutation of its ids);
  3. q, then K of every token, then V of every token, each N(0, 1) in float32,
     rounded to the storage dtype with round-to-nearest-even.

Token order for K and V: all shared-prompt tokens (prompt 0 first, positions in
order), then every sequence's private tokens (sequence 0 first).  The last
private token of a sequence is the token being decoded.

Storage dtypes are passed around as raw bits: ``uint16`` for bf16 and fp16,
``float32`` for fp32.  Nothing here builds block tables, slots or attention;
both the oracle and the HIP path do that themselves from these inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
_CHUNK = 1 << 22  # values per draw (the stream does not depend on it)

CONFIG_NAMES = {
    1: "tiny-f32",
    2: "llama3-8b-layer-bf16",
    3: "llama3-70b-layer-mixed-bf16",
    4: "shared-prefix-n4-bf16",
    5: "long-context-32k-f16",
    # variant of 4: one prefix shared by all 256 sequences
    "4b": "shared-prefix-all-bf16",
    # chunked prefill: 16 sequences, a 512-token chunk each after U{0..3584}
    # cached tokens, Llama-3-8B layer shape
    "prefill": "chunked-prefill-8b-bf16",
}


def bits_dtype(dtype: str):
    """numpy dtype that carries the storage bits of ``dtype``."""
    if dtype == "f32":
        return np.dtype(np.float32)
    if dtype in ("bf16", "f16"):
        return np.dtype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def elem_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def round_to_dtype_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage bits of ``dtype``, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        if not np.all(np.isfinite(x)):
            raise ValueError("bf16 rounding here handles finite values only")
        b = x.view(np.uint32).astype(np.uint64)
        b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
        return b.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class Workload:
    """One decode batch: shapes, sequence structure, pool order and values."""

    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    scale: float
    num_blocks: int
    free_order: np.ndarray  # int32 [num_blocks], a permutation of range(num_blocks)
    prompt_of: np.ndarray  # int32 [S]; -1 = the sequence has no shared prompt
    prompt_lens: np.ndarray  # int32 [P]
    private_lens: np.ndarray  # int32 [S]; >= 1, the last one is being decoded
    step_lens: np.ndarray  # int32 [S]; trailing tokens written by the measured step
    q: np.ndarray  # bits [S, Hq, D]
    k_prompt: np.ndarray  # bits [sum(prompt_lens), Hkv, D]
    v_prompt: np.ndarray
    k_private: np.ndarray  # bits [sum(private_lens), Hkv, D]
    v_private: np.ndarray
    block_size: int = BLOCK_SIZE
    notes: dict = field(default_factory=dict)
    # chunked prefill: one query per token the step writes, [sum(step_lens), Hq, D]
    chunk_q: np.ndarray | None = None

    @property
    def query_start(self) -> np.ndarray:
        """Row offsets of each sequence's chunk in ``chunk_q`` (int32 [S + 1])."""
        return np.concatenate([[0], np.cumsum(self.step_lens, dtype=np.int64)]).astype(np.int32)

    # ---- bookkeeping helpers (index arithmetic over the arrays above) ----
    @property
    def num_seqs(self) -> int:
        return int(self.private_lens.shape[0])

    @property
    def context_lens(self) -> np.ndarray:
        """Length of every sequence including the token being decoded."""
        pl = np.zeros(self.num_seqs, dtype=np.int64)
        has = self.prompt_of >= 0
        pl[has] = self.prompt_lens[self.prompt_of[has]]
        return (pl + self.private_lens).astype(np.int32)

    @property
    def prompt_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.prompt_lens, dtype=np.int64)])

    @property
    def private_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.private_lens, dtype=np.int64)])

    @property
    def elem_bytes(self) -> int:
        return elem_bytes(self.dtype)

    def int8_scales(self):
        """Per-channel scales (k_scale, v_scale), float32 [Hkv, D], of an INT8
        cache of this workload: (3.5 + U[0, 1)) / 127, so that codes saturate
        only beyond 3.5-4.5 standard deviations of the N(0, 1) values.  Drawn
        from their own stream (seed, 8), leaving every other draw unchanged."""
        rng = np.random.default_rng([int(self.seed), 8])
        shape = (self.num_kv_heads, self.head_dim)
        k = ((3.5 + rng.random(shape)) / 127).astype(np.float32)
        v = ((3.5 + rng.random(shape)) / 127).astype(np.float32)
        return k, v

    def prompt_tokens(self, p: int) -> np.ndarray:
        """Token ids of shared prompt ``p`` (int32): id = p * 2**16 + position.
        The K/V drawn for a prompt token belong to that id alone, so a prefix
        cache keyed on ids may share them."""
        return (int(p) * 65536 + np.arange(int(self.prompt_lens[p]))).astype(np.int32)

    def sequence_kv(self, s: int):
        """Contiguous (K, V) bits of sequence ``s``, positions 0..len-1."""
        parts_k, parts_v = [], []
        p = int(self.prompt_of[s])
        if p >= 0:
            a, b = self.prompt_offsets[p], self.prompt_offsets[p + 1]
            parts_k.append(self.k_prompt[a:b])
            parts_v.append(self.v_prompt[a:b])
        a, b = self.private_offsets[s], self.private_offsets[s + 1]
        parts_k.append(self.k_private[a:b])
        parts_v.append(self.v_private[a:b])
        return np.concatenate(parts_k), np.concatenate(parts_v)


def _normal_bits(rng, n: int, dtype: str) -> np.ndarray:
    """n draws of N(0, 1) in float32, rounded to ``dtype`` (reused buffers)."""
    out = np.empty(n, dtype=bits_dtype(dtype))
    buf = np.empty(min(n, _CHUNK), dtype=np.float32)
    tmp = np.empty(min(n, _CHUNK), dtype=np.uint32)
    for a in range(0, n, _CHUNK):
        b = min(n, a + _CHUNK)
        x, t = buf[:b - a], tmp[:b - a]
        rng.standard_normal(out=x, dtype=np.float32)
        if dtype == "f32":
            out[a:b] = x
        elif dtype == "f16":
            out.view(np.float16)[a:b] = x  # round to nearest even
        else:  # bf16: add 0x7FFF plus the kept LSB, keep the high half
            u = x.view(np.uint32)
            np.right_shift(u, 16, out=t)
            np.bitwise_and(t, 1, out=t)
            t += 0x7FFF
            t += u
            t >>= 16
            out[a:b] = t
    return out


def _build(name, seed, rng, *, hq, hkv, d, dtype, prompt_of, prompt_lens,
           private_lens, num_blocks, step_lens=None, scale=None, notes=None,
           values=True) -> Workload:
    prompt_of = np.asarray(prompt_of, dtype=np.int32)
    prompt_lens = np.asarray(prompt_lens, dtype=np.int32)
    private_lens = np.asarray(private_lens, dtype=np.int32)
    if np.any(private_lens < 1):
        raise ValueError("every sequence owns at least the token being decoded")
    if step_lens is None:
        step_lens = np.ones_like(private_lens)
    step_lens = np.asarray(step_lens, dtype=np.int32)
    if np.any(step_lens < 1) or np.any(step_lens > private_lens):
        raise ValueError("the step writes 1..private_len trailing tokens")
    free_order = rng.permutation(num_blocks).astype(np.int32)
    s = private_lens.shape[0]
    n_prompt = int(prompt_lens.sum())
    n_priv = int(private_lens.sum())
    if values:
        q = _normal_bits(rng, s * hq * d, dtype).reshape(s, hq, d)
        k = _normal_bits(rng, (n_prompt + n_priv) * hkv * d, dtype).reshape(-1, hkv, d)
        v = _normal_bits(rng, (n_prompt + n_priv) * hkv * d, dtype).reshape(-1, hkv, d)
    else:  # structure only: zero-filled values of the right shapes (no draws)
        q = np.zeros((s, hq, d), dtype=bits_dtype(dtype))
        k = np.broadcast_to(np.zeros((1, 1, 1), bits_dtype(dtype)), (n_prompt + n_priv, hkv, d))
        v = k
    return Workload(
        name=name, seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        dtype=dtype, scale=float(1.0 / math.sqrt(d)) if scale is None else float(scale),
        num_blocks=int(num_blocks), free_order=free_order, prompt_of=prompt_of,
        prompt_lens=prompt_lens, private_lens=private_lens, step_lens=step_lens, q=q,
        k_prompt=k[:n_prompt], v_prompt=v[:n_prompt],
        k_private=k[n_prompt:], v_private=v[n_prompt:], notes=dict(notes or {}))


def _ceil_div(a, b):
    return -(-np.asarray(a, dtype=np.int64) // b)


def _pool_size_unshared(lens, factor=1.1):
    # Pool sizing rule of the workloads: 1.1x the blocks the batch occupies.
    return int(math.ceil(factor * int(_ceil_div(lens, BLOCK_SIZE).sum())))


def make_prefill(chunk_lens, cached_lens, *, hq, hkv, d, dtype, seed=0, name="prefill-custom",
                 num_blocks=None) -> Workload:
    """Chunked-prefill batch: sequence s holds cached_lens[s] tokens and
    appends a chunk of chunk_lens[s] >= 1 tokens in the step; ``chunk_q``
    holds one query per chunk token, drawn after everything else."""
    chunk_lens = np.asarray(chunk_lens, dtype=np.int32)
    lens = np.asarray(cached_lens, dtype=np.int32) + chunk_lens
    rng = np.random.Generator(np.random.PCG64(seed))
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(1.25 * _pool_size_unshared(lens, 1.0))) + 2)
    w = _build(name, seed, rng, hq=hq, hkv=hkv, d=d, dtype=dtype,
               prompt_of=-np.ones(lens.shape[0], np.int32), prompt_lens=[], private_lens=lens,
               num_blocks=num_blocks, step_lens=chunk_lens)
    w.chunk_q = _normal_bits(rng, int(chunk_lens.sum()) * hq * d, dtype).reshape(-1, hq, d)
    return w


def make(config, seed=None, values=True) -> Workload:
    """Workload ``config`` (1..5 or "4b") with its own seed unless one is given.

    ``values=False`` skips the value draws (structure and pool order are drawn
    first, so they are the same either way).
    """
    key = config
    if isinstance(config, str) and config.isdigit():
        key = int(config)
    if key not in CONFIG_NAMES:
        raise ValueError(f"unknown workload {config!r}")
    if key == "prefill":
        seed = 6 if seed is None else int(seed)
        rng = np.random.Generator(np.random.PCG64(seed))
        cached = rng.integers(0, 3584, size=16, endpoint=True).astype(np.int32)
        w = make_prefill(np.full(16, 512, np.int32), cached, hq=32, hkv=8, d=128, dtype="bf16",
                         seed=seed + 1000, name=CONFIG_NAMES[key])
        w.seed = seed
        return w
    seed = (4 if key == "4b" else int(key)) if seed is None else int(seed)
    rng = np.random.Generator(np.random.PCG64(seed))
    name = CONFIG_NAMES[key]

    if key == 1:
        lens = np.array([1, 17, 33, 100], dtype=np.int32)
        return _build(name, seed, rng, hq=4, hkv=2, d=64, dtype="f32", values=values,
                      prompt_of=-np.ones(4, np.int32), prompt_lens=[], private_lens=lens,
                      num_blocks=64)
    if key == 2:
        lens = rng.integers(128, 4096, size=64, endpoint=True).astype(np.int32)
        return _build(name, seed, rng, hq=32, hkv=8, d=128, dtype="bf16", values=values,
                      prompt_of=-np.ones(64, np.int32), prompt_lens=[], private_lens=lens,
                      num_blocks=_pool_size_unshared(lens))
    if key == 3:
        x = rng.lognormal(mean=math.log(300.0), sigma=1.0, size=256)
        lens = np.clip(np.rint(x), 16, 8192).astype(np.int32)
        return _build(name, seed, rng, hq=64, hkv=8, d=128, dtype="bf16", values=values,
                      prompt_of=-np.ones(256, np.int32), prompt_lens=[], private_lens=lens,
                      num_blocks=_pool_size_unshared(lens))
    if key in (4, "4b"):
        n_prompts, n = (64, 4) if key == 4 else (1, 256)
        tails = rng.integers(1, 15, size=n_prompts, endpoint=True)
        prompt_lens = (2048 + tails).astype(np.int32)
        private = rng.integers(1, 300, size=n_prompts * n, endpoint=True).astype(np.int32)
        prompt_of = np.repeat(np.arange(n_prompts, dtype=np.int32), n)
        # upper bound of the blocks the batch occupies: every prompt once, and
        # every sample from the start of its prompt's partial block onwards
        est = int(_ceil_div(prompt_lens, BLOCK_SIZE).sum())
        est += int(_ceil_div(prompt_lens[prompt_of] % BLOCK_SIZE + private, BLOCK_SIZE).sum())
        return _build(name, seed, rng, hq=32, hkv=8, d=128, dtype="bf16", values=values,
                      prompt_of=prompt_of, prompt_lens=prompt_lens, private_lens=private,
                      step_lens=private, num_blocks=int(math.ceil(1.1 * est)),
                      notes={"samples_per_prompt": n})
    if key == 5:
        lens = np.full(8, 32768, dtype=np.int32)
        return _build(name, seed, rng, hq=64, hkv=8, d=128, dtype="f16", values=values,
                      prompt_of=-np.ones(8, np.int32), prompt_lens=[], private_lens=lens,
                      num_blocks=_pool_size_unshared(lens),
                      notes={"partition_size": 512})
    raise AssertionError


def make_custom(lens, *, hq, hkv, d, dtype, seed=0, num_blocks=None, scale=None,
                prompt_lens=None, prompt_of=None, step_lens=None,
                name="custom") -> Workload:
    """Ad-hoc workload for tests.

    ``lens`` are the private lengths (the full context lengths when there is no
    shared prompt).  With ``prompt_lens``/``prompt_of`` given, sequence s is
    prompt ``prompt_of[s]`` followed by ``lens[s]`` private tokens.  ``step_lens``
    defaults to 1 (only the decoded token) without prompts, and to every private
    token with them (so that the step is where the samples diverge).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(lens, dtype=np.int32)
    if prompt_lens is None:
        prompt_lens = np.zeros(0, np.int32)
        prompt_of = -np.ones(lens.shape[0], np.int32)
        total = _pool_size_unshared(lens, 1.0)
    else:
        prompt_lens = np.asarray(prompt_lens, np.int32)
        prompt_of = np.asarray(prompt_of, np.int32)
        total = int(_ceil_div(prompt_lens, BLOCK_SIZE).sum())
        total += int(_ceil_div(lens, BLOCK_SIZE).sum()) + lens.shape[0]
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(1.25 * total)) + 2)
    if step_lens is None and np.any(prompt_of >= 0):
        step_lens = lens
    return _build(name, seed, rng, hq=hq, hkv=hkv, d=d, dtype=dtype,
                  prompt_of=prompt_of, prompt_lens=prompt_lens, private_lens=lens,
                  num_blocks=num_blocks, step_lens=step_lens, scale=scale)
