"""paged_attention_decode on the GPU against the oracle.

Every case compares every output with the oracle's paged decode (tables and
cache built by the oracle itself from the same seeded inputs): small shape
cases, and the five workloads at full size in the launch configuration the
benchmark times (the long-context workload also at its stated split of 512
positions).  Properties that hold at any size (split == unsplit, run-to-run
and block-relabelling invariance) are checked beside them.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_06_amd as pa
import workloads
from oracle import step
from oracle.numerics import to_f64
from paged_kv_cache_06_amd import runner
from tests.helpers import NAN_BITS, assert_close, bits_of

pytestmark = pytest.mark.gpu


def _run_small(w, partition_size=pa.PARTITION_AUTO, prefix_cache=False):
    ref_plan, kc, vc, ref = step.run(w, NAN_BITS[w.dtype], prefix_cache=prefix_cache)
    db = runner.DeviceBatch(w, prefix_cache=prefix_cache)
    db.prefill()
    db.step(partition_size=partition_size)
    return db, ref


CASES = [
    # (lens, hq, hkv, d, dtype)
    ([1, 15, 16, 17, 33, 100, 257, 600], 8, 2, 128, "bf16"),
    ([1, 15, 16, 17, 33, 100, 257, 600], 8, 2, 128, "f16"),
    ([3, 64, 129, 700, 1100], 16, 2, 64, "bf16"),
    ([5, 48, 511, 512, 513, 1025], 32, 8, 128, "bf16"),   # G = 4
    ([7, 100, 300], 64, 8, 128, "bf16"),                    # G = 8
    ([9, 200], 32, 1, 128, "f16"),                          # MQA, G = 32 (2 head blocks)
    ([9, 300, 1100], 64, 1, 128, "bf16"),                   # MQA, G = 64 (4 head blocks)
    ([31, 90], 4, 4, 128, "bf16"),                          # MHA, G = 1
    ([5, 77, 400], 4, 2, 64, "f16"),                        # G = 2
    ([20, 300, 1000], 12, 4, 128, "bf16"),                  # G = 3 (4-row head group)
    ([1, 17, 33, 100], 4, 2, 64, "f32"),                    # generic VALU path
    ([2, 40, 700], 8, 2, 32, "bf16"),                       # generic path, D = 32
    ([2, 40, 300], 4, 2, 256, "f16"),                       # generic path, D = 256
    ([20, 1000], 12, 4, 96, "f32"),                         # generic path, D = 96, G = 3
    # 40 sequences at 8 KV heads: at partitions of 16 and 64 the work list is
    # longer than the decode grid, so the plan doubles the partition size
    (list(range(600, 1000, 10)), 32, 8, 64, "bf16"),
]


@pytest.mark.parametrize("lens,hq,hkv,d,dtype", CASES)
@pytest.mark.parametrize("partition_size", [pa.PARTITION_AUTO, pa.PARTITION_NONE, 16, 64, 512])
def test_small_cases_against_oracle(lens, hq, hkv, d, dtype, partition_size):
    print(f"[gpu] decode lens={lens} hq={hq} hkv={hkv} d={d} {dtype} P={partition_size}",
          flush=True)
    w = workloads.make_custom(lens, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=sum(lens) + hq)
    db, ref = _run_small(w, partition_size)
    assert_close(db.out_bits(), ref, dtype, f"{lens} {hq}/{hkv} d={d} {dtype}")


EIGHT_WAVE_CASES = [
    # (hq, hkv, d, dtype): 8 waves per item at D 64, and at D 128 up to 15
    # query heads per KV head; 16 or more at D 128 fall back to 4 waves
    (16, 2, 128, "bf16"),   # G = 8: 8 waves
    (16, 2, 64, "f16"),     # G = 8: 8 waves
    (32, 2, 64, "bf16"),    # G = 16, D 64: 8 waves, a full 16-head block
    (32, 2, 128, "bf16"),   # G = 16, D 128: 4 waves (8 waves' partials exceed 64 KiB)
    (64, 2, 128, "f16"),    # G = 32: 4 waves, 2 head blocks
    (64, 1, 128, "bf16"),   # G = 64: 4 waves, 4 head blocks
]


@pytest.mark.parametrize("hq,hkv,d,dtype", EIGHT_WAVE_CASES)
@pytest.mark.parametrize("partition_size", [pa.PARTITION_AUTO, 2048, 4096])
def test_long_context_items_against_oracle(hq, hkv, d, dtype, partition_size):
    # a batch whose longest context passes 16K positions: partitions of >= 2048
    # positions run the items kernel with 8 waves per work-group where the
    # partials fit the LDS, 4 otherwise
    print(f"[gpu] long-context items hq={hq} hkv={hkv} d={d} {dtype} P={partition_size}",
          flush=True)
    lens = [17, 100, 2100, 4500, 16500]
    w = workloads.make_custom(lens, hq=hq, hkv=hkv, d=d, dtype=dtype,
                              seed=hq + d + max(partition_size, 0))
    db, ref = _run_small(w, partition_size)
    assert_close(db.out_bits(), ref, dtype,
                 f"long context {hq}/{hkv} {d} {dtype} P={partition_size}")


def test_tiny_config_every_output():
    print("[gpu] workload 1 (tiny fp32)", flush=True)
    w = workloads.make(1)
    db, ref = _run_small(w)
    assert_close(db.out_bits(), ref, "f32", "tiny")


def test_shared_prefix_small_against_oracle():
    print("[gpu] shared prefix small", flush=True)
    w = workloads.make_custom([1, 5, 20, 2, 3, 40, 7, 9], hq=8, hkv=2, d=128, dtype="bf16",
                              seed=8, prompt_lens=[21, 32, 45], prompt_of=[0, 0, 0, 1, 1, 1, 2, 2])
    db, ref = _run_small(w)
    assert_close(db.out_bits(), ref, "bf16", "shared prefix")


def test_shared_prefix_small_through_prefix_cache_against_oracle():
    print("[gpu] shared prefix small, prefix cache", flush=True)
    w = workloads.make_custom([1, 5, 20, 2, 3, 40, 7, 9], hq=8, hkv=2, d=128, dtype="bf16",
                              seed=8, prompt_lens=[21, 32, 45], prompt_of=[0, 0, 0, 1, 1, 1, 2, 2])
    db, ref = _run_small(w, prefix_cache=True)
    assert db.bm.pool.stats()["prefix_hits"] > 0
    assert_close(db.out_bits(), ref, "bf16", "shared prefix, prefix cache")


def test_zero_length_rows_give_zeros_and_others_unaffected():
    import torch
    print("[gpu] zero-length rows", flush=True)
    w = workloads.make_custom([40, 70, 1], hq=8, hkv=2, d=128, dtype="bf16", seed=2)
    db, ref = _run_small(w)
    lens = db.context_lens.clone()
    lens[1] = 0
    out = torch.full_like(db.out, float("nan"))
    kc, vc = db.caches[0]
    pa.paged_attention_decode(db.q, kc, vc, db.tables, lens, w.scale, out,
                              max_context_len=db.max_context_len)
    got = bits_of(out)
    assert np.all(to_f64(got[1], "bf16") == 0)
    assert np.array_equal(got[[0, 2]], db.out_bits()[[0, 2]])


def test_many_sequences():
    # more sequences than threads of the plan kernel: several per thread
    print("[gpu] 1100 sequences", flush=True)
    lens = (np.arange(1100) % 45) + 1
    w = workloads.make_custom(lens, hq=8, hkv=2, d=64, dtype="bf16", seed=5)
    db, ref = _run_small(w, 16)
    assert_close(db.out_bits(), ref, "bf16", "1100 sequences")


@pytest.mark.parametrize("partition_size", [pa.PARTITION_AUTO, 16])
def test_more_sequences_than_the_plan_stages_in_lds(partition_size):
    # above 4096 sequences the plan reads the lengths from global memory
    # instead of its LDS copy, 20 sequences per plan thread
    print(f"[gpu] 5000 sequences P={partition_size}", flush=True)
    lens = (np.arange(5000) * 7 % 61) + 1
    w = workloads.make_custom(lens, hq=4, hkv=1, d=64, dtype="bf16", seed=11)
    db, ref = _run_small(w, partition_size)
    assert_close(db.out_bits(), ref, "bf16", "5000 sequences")


@pytest.mark.parametrize("config,expect", [("2", 2048), ("5", 4096), ("3", 1024)])
def test_even_batches_double_the_automatic_partition(config, expect):
    # the plan doubles an automatic partition for a batch of evenly long
    # sequences (8B layer 1024 -> 2048, 32K context 2048 -> 4096) and keeps
    # it for the skewed mixed batch; a partition the caller passes is kept.
    # The outputs at the doubled partition are checked against the oracle by
    # the full-size tests.
    print(f"[gpu] even-batch partition, workload {config}", flush=True)
    db = runner.DeviceBatch(workloads.make(config))
    db.prefill()
    db.step()
    assert pa.last_plan_partition() == expect
    db.step(partition_size=1024)
    assert pa.last_plan_partition() == 1024


def test_stale_workspace_does_not_matter():
    # the workspace is scratch: a NaN-filled one and a reused one give the same bits
    import torch
    print("[gpu] stale workspace", flush=True)
    w = workloads.make_custom([5, 300, 1000, 2], hq=8, hkv=2, d=128, dtype="bf16", seed=3)
    db, ref = _run_small(w, 64)
    kc, vc = db.caches[0]
    need = pa.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.head_dim, db.max_context_len, 64)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    for _ in range(3):
        out = torch.empty_like(db.out)
        pa.paged_attention_decode(db.q, kc, vc, db.tables, db.context_lens, w.scale, out,
                                  max_context_len=db.max_context_len, partition_size=64,
                                  workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), db.out_bits())


def test_timing_records_every_launch():
    print("[gpu] timing launch list", flush=True)
    w = workloads.make_custom([5, 300, 1000, 2], hq=8, hkv=2, d=128, dtype="bf16", seed=4)
    db, _ = _run_small(w, 64)
    kc, vc = db.caches[0]
    pa.timing_begin(16)
    for _ in range(3):
        pa.paged_attention_decode(db.q, kc, vc, db.tables, db.context_lens, w.scale,
                                  torch.empty_like(db.out), max_context_len=db.max_context_len,
                                  partition_size=64)
    torch.cuda.synchronize()
    kt = pa.timing_end()
    ms = pa.timing_launches("decode")
    assert kt["decode"]["launches"] == 3 and len(ms) == 3
    assert all(v > 0 for v in ms)
    assert abs(sum(ms) - kt["decode"]["ms"]) <= 1e-9 * max(1.0, kt["decode"]["ms"])
    assert len(pa.timing_launches("decode_plan")) == 3


def test_nan_in_table_padding_and_block_tails_does_not_leak():
    # every unused table entry points at a NaN block, every unwritten slot is NaN;
    # a clean run on a zero-filled cache must give the same bits
    print("[gpu] poison", flush=True)
    w = workloads.make_custom([1, 17, 35, 190], hq=16, hkv=2, d=128, dtype="f16", seed=12)
    a = runner.DeviceBatch(w)
    a.prefill()
    a.step()
    b = runner.DeviceBatch(w, fill=0.0)
    b.prefill()
    b.step()
    assert np.all(np.isfinite(to_f64(a.out_bits(), "f16")))
    assert np.array_equal(a.out_bits(), b.out_bits())


# ---- full-size workloads, in the benchmark's launch configuration ----

_FULL = {}
_ORACLE = {}


def _full(config):
    """The workload on the device after the benchmark's step (copies, token
    writes, decode with the automatic partition); one workload kept at a time."""
    if config not in _FULL:
        _FULL.clear()
        import torch
        w = workloads.make(config)
        db = runner.DeviceBatch(w)
        db.prefill()
        db.step()
        torch.cuda.synchronize()
        _FULL[config] = (w, db)
    return _FULL[config]


def _oracle_full(config):
    """The oracle's run of the same workload: (plan, k_cache, v_cache, out)."""
    if config not in _ORACLE:
        _ORACLE.clear()
        w, _ = _full(config)
        _ORACLE[config] = step.run(w, NAN_BITS[w.dtype])
    return _ORACLE[config]


@pytest.mark.parametrize("config", [2, 3, 4, 5])
def test_full_size_every_output_against_oracle(config):
    print(f"[gpu] full-size workload {config}: every output against the oracle", flush=True)
    w, db = _full(config)
    _, _, _, ref = _oracle_full(config)
    info = assert_close(db.out_bits(), ref, w.dtype, f"workload {config}")
    print(f"  {w.num_seqs} sequences x {w.num_q_heads} heads: {info}", flush=True)


def test_full_size_long_context_at_its_stated_split():
    # the long-context workload names split-K partitions of 512 positions
    # plus a reduce: every output of that launch against the oracle
    import torch
    print("[gpu] full-size workload 5 at partitions of 512: every output", flush=True)
    w, db = _full(5)
    _, _, _, ref = _oracle_full(5)
    out = torch.full_like(db.out, float("nan"))
    db.decode(partition_size=512, out=out)
    torch.cuda.synchronize()
    info = assert_close(bits_of(out), ref, w.dtype, "workload 5, P = 512")
    print(f"  {info}", flush=True)


@pytest.mark.parametrize("config", [3, 5])
def test_full_size_split_equals_unsplit_and_is_deterministic(config):
    import torch
    print(f"[gpu] full-size workload {config}: split/unsplit/determinism", flush=True)
    w, db = _full(config)
    base = db.out_bits()
    out2 = torch.empty_like(db.out)
    db.decode(partition_size=pa.PARTITION_AUTO, out=out2)
    assert np.array_equal(bits_of(out2), base)  # run to run
    b = to_f64(base, w.dtype)
    # the splits differ in summation order and in the running maxima the
    # weights are taken against; a weight enters the matrix core as a hi + lo
    # pair in the storage dtype, exact to about 2^-16 of itself, so outputs
    # that nearly cancel can move by ~1e-6 in absolute terms.  After rounding
    # to the storage dtype the results are at most one unit in its last place
    # apart, or 1e-5 where the output is that small.
    ulp = 2.0 ** -7 if w.dtype == "bf16" else 2.0 ** -10
    for ps in (pa.PARTITION_NONE, 256, 512, 1024):
        db.decode(partition_size=ps, out=out2)
        c = to_f64(bits_of(out2), w.dtype)
        ratio = np.abs(c - b) / (ulp * np.abs(b) + 1e-5)
        assert ratio.max() <= 1.0, f"partition {ps}: {ratio.max():.2f} ulp"


def test_full_size_block_relabelling_is_bit_identical():
    print("[gpu] full-size workload 3: relabelled blocks", flush=True)
    w, db = _full(3)
    base = db.out_bits()
    w2 = workloads.make(3)
    w2.free_order = np.random.default_rng(99).permutation(w2.num_blocks).astype(np.int32)
    db2 = runner.DeviceBatch(w2)
    db2.prefill()
    db2.step()
    assert not np.array_equal(db2.bm.rows, db.bm.rows)
    assert np.array_equal(db2.out_bits(), base)


def test_full_size_shared_prefix_through_cache_is_bit_identical_to_forks():
    print("[gpu] full-size workload 4: prefix cache vs forks", flush=True)
    w, db = _full(4)
    base = db.out_bits()
    db2 = runner.DeviceBatch(w, prefix_cache=True)
    db2.prefill()
    db2.step()
    assert not np.array_equal(db2.bm.rows, db.bm.rows)
    assert db2.bm.pool.stats()["prefix_hits"] == 64 * 3 * 128
    assert np.array_equal(db2.out_bits(), base)


@pytest.mark.parametrize("dtype,d,partition_size", [("bf16", 128, pa.PARTITION_AUTO),
                                                    ("f16", 64, 64),
                                                    ("bf16", 128, pa.PARTITION_NONE),
                                                    ("f32", 64, pa.PARTITION_AUTO)])
def test_fused_step_equals_write_then_decode(dtype, d, partition_size):
    """decode_step (token writes in the plan's launch where it can) against
    reshape_and_cache followed by paged_attention_decode: same cache bits,
    same outputs, bit for bit."""
    import torch
    print(f"[gpu] fused step {dtype} D={d} P={partition_size}", flush=True)
    w = workloads.make_custom([1, 5, 20, 2, 3, 40, 700, 9], hq=8, hkv=2, d=d, dtype=dtype,
                              seed=31, prompt_lens=[21, 32, 45],
                              prompt_of=[0, 0, 0, 1, 1, 1, 2, 2])
    a = runner.DeviceBatch(w)
    b = runner.DeviceBatch(w)
    for db, fused in ((a, True), (b, False)):
        db.prefill()
        db.step(partition_size=partition_size, fused=fused)
    torch.cuda.synchronize()
    for x, y in zip(a.caches[0], b.caches[0]):
        assert torch.equal(x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32),
                           y.view(torch.int16) if y.element_size() == 2 else y.view(torch.int32))
    assert np.array_equal(a.out_bits(), b.out_bits())
    _, _, _, ref = step.run(w, NAN_BITS[dtype])
    assert_close(a.out_bits(), ref, dtype, "fused step")
