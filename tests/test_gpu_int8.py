"""INT8 KV cache on the GPU against the oracle (oracle.quant).

Codes written by reshape_and_cache_int8 are compared bit for bit with the
oracle's quantization (the integer decision is taken in fp32 on both sides);
decode over the INT8 cache is compared with the oracle's fp64 attention over
the values code * scale, at the tolerance of the 16-bit path.
"""
import numpy as np
import pytest

import paged_kv_cache_06_amd as pa
import workloads
from oracle import quant, step
from oracle.numerics import to_f64
from paged_kv_cache_06_amd import runner
from tests.helpers import assert_close, bits_of

pytestmark = pytest.mark.gpu


def _codes(db, copy=0):
    k, v = pa.logical_view(*db.caches[copy])
    return k.cpu().numpy(), v.cpu().numpy()


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f32", 128)])
def test_cache_writes_and_copies_are_bit_exact(dtype, d):
    print(f"[gpu] int8 cache writes {dtype} D={d}", flush=True)
    w = workloads.make_custom([1, 5, 20, 2, 3, 40, 7, 9], hq=8, hkv=2, d=d, dtype=dtype,
                              seed=21, prompt_lens=[21, 32, 45],
                              prompt_of=[0, 0, 0, 1, 1, 1, 2, 2])
    pl, kc, vc, _ = step.run_int8(w)
    assert sum(len(ph.pairs) for ph in pl.phases) > 0  # copies on the INT8 cache too
    db = runner.DeviceBatch(w, int8=True)
    db.prefill()
    db._apply(db.dev_phases[2], db.caches[0])
    k, v = _codes(db)
    nb = w.num_blocks
    assert np.array_equal(k[:nb], kc) and np.array_equal(v[:nb], vc)
    assert np.all(k[nb] == 127) and np.all(v[nb] == 127)  # poison block untouched


def test_special_values_quantize_like_the_oracle():
    import torch
    print("[gpu] int8 special values", flush=True)
    hkv, d, t = 2, 64, 6
    rng = np.random.default_rng(3)
    sk = np.full((hkv, d), 2.0 ** -5, np.float32)  # x / s exact: ties stay ties
    sv = rng.uniform(0.01, 0.05, (hkv, d)).astype(np.float32)
    x = (rng.integers(-300, 300, (t, hkv, d)) * 0.5 * 2.0 ** -5).astype(np.float32)
    x[0, 0, :8] = [np.nan, np.inf, -np.inf, 0.5 * 2 ** -5, 1.5 * 2 ** -5, -2.5 * 2 ** -5, 1e30, -0.0]
    y = rng.standard_normal((t, hkv, d)).astype(np.float32) * 3
    kq, vq = pa.new_kv_cache_int8(4, hkv, d, "cuda", 33)
    slots = np.array([0, 17, -1, 63, 40, 5], np.int64)
    pa.reshape_and_cache_int8(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda(), kq, vq,
                              torch.from_numpy(slots).cuda(), torch.from_numpy(sk).cuda(),
                              torch.from_numpy(sv).cuda())
    kc = np.full((4, hkv, 16, d), 33, np.int8)
    vc = kc.copy()
    quant.reshape_and_cache(x, y, "f32", kc, vc, slots, sk, sv)
    k, v = pa.logical_view(kq, vq)
    assert np.array_equal(k.cpu().numpy(), kc) and np.array_equal(v.cpu().numpy(), vc)
    assert kc[0, 0, 0, :8].tolist() == [0, 127, -127, 0, 2, -2, 127, 0]


def test_near_ties_at_general_scales_quantize_like_the_oracle():
    # scales that are not powers of two: the writer's fast quotient x * rcp(s)
    # decides far from a tie and the exact fp32 division near one; planted
    # values are the fp32 ties (k + 1/2) * s and their neighbours one ulp away
    import torch
    print("[gpu] int8 near-ties at general scales", flush=True)
    hkv, d, t = 2, 128, 64
    rng = np.random.default_rng(17)
    sk = ((3.5 + rng.random((hkv, d))) / 127).astype(np.float32)
    sv = rng.uniform(1e-3, 0.2, (hkv, d)).astype(np.float32)
    k = rng.integers(-130, 130, (t, hkv, d)).astype(np.float32)
    tie = ((k + np.float32(0.5)) * sk).astype(np.float32)
    step_ = rng.integers(-1, 2, (t, hkv, d))  # the tie, or one ulp below or above it
    x = np.where(step_ == 0, tie, np.nextafter(tie, np.where(step_ > 0, np.inf, -np.inf)))
    x = x.astype(np.float32)
    y = (rng.standard_normal((t, hkv, d)) * 10).astype(np.float32)
    kq, vq = pa.new_kv_cache_int8(8, hkv, d, "cuda", 33)
    slots = rng.permutation(8 * 16)[:t].astype(np.int64)
    pa.reshape_and_cache_int8(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda(), kq, vq,
                              torch.from_numpy(slots).cuda(), torch.from_numpy(sk).cuda(),
                              torch.from_numpy(sv).cuda())
    kc = np.full((8, hkv, 16, d), 33, np.int8)
    vc = kc.copy()
    quant.reshape_and_cache(x, y, "f32", kc, vc, slots, sk, sv)
    kg, vg = pa.logical_view(kq, vq)
    assert np.array_equal(kg.cpu().numpy(), kc) and np.array_equal(vg.cpu().numpy(), vc)


CASES = [
    # (lens, hq, hkv, d, dtype)
    ([1, 15, 16, 17, 33, 100, 257, 600], 8, 2, 128, "bf16"),
    ([1, 15, 16, 17, 33, 100, 257, 600], 8, 2, 128, "f16"),
    ([3, 64, 129, 700, 1100], 16, 2, 64, "bf16"),
    ([7, 100, 300], 64, 8, 128, "bf16"),                    # G = 8
    ([9, 200], 32, 1, 128, "f16"),                          # MQA, 2 head blocks
    ([9, 300, 1100], 64, 1, 64, "bf16"),                    # MQA, 4 head blocks
    ([31, 90], 4, 4, 64, "bf16"),                           # MHA
    ([20, 300, 1000], 12, 4, 128, "bf16"),                  # G = 3
    (list(range(600, 1000, 10)), 32, 8, 64, "bf16"),       # partition doubled by the plan
]


@pytest.mark.parametrize("lens,hq,hkv,d,dtype", CASES)
@pytest.mark.parametrize("partition_size", [pa.PARTITION_AUTO, pa.PARTITION_NONE, 16, 64, 512])
def test_small_cases_against_oracle(lens, hq, hkv, d, dtype, partition_size):
    print(f"[gpu] int8 decode {lens} {hq}/{hkv} D={d} {dtype} P={partition_size}", flush=True)
    w = workloads.make_custom(lens, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=len(lens) + d)
    _, _, _, ref = step.run_int8(w)
    db = runner.DeviceBatch(w, int8=True)
    db.prefill()
    db.step(partition_size=partition_size)
    assert_close(db.out_bits(), ref, dtype, f"int8 {lens} P={partition_size}")


@pytest.mark.parametrize("hq,hkv,d", [(16, 2, 128), (32, 2, 64), (32, 2, 128), (64, 2, 128),
                                      (64, 1, 128)])
@pytest.mark.parametrize("partition_size", [pa.PARTITION_AUTO, 4096, 8192])
def test_long_context_items_against_oracle(hq, hkv, d, partition_size):
    # a batch whose longest context passes 16K positions: INT8 partitions of
    # >= 4096 positions run with 8 waves per work-group where the partials fit
    # the LDS (G <= 15 at D 128, G <= 16 at D 64), 4 otherwise
    print(f"[gpu] int8 long-context items {hq}/{hkv} D={d} P={partition_size}", flush=True)
    lens = [17, 100, 4200, 16500]
    w = workloads.make_custom(lens, hq=hq, hkv=hkv, d=d, dtype="bf16",
                              seed=hq + d + max(partition_size, 0))
    _, _, _, ref = step.run_int8(w)
    db = runner.DeviceBatch(w, int8=True)
    db.prefill()
    db.step(partition_size=partition_size)
    assert_close(db.out_bits(), ref, "bf16", f"int8 long context {hq}/{hkv} P={partition_size}")


def test_shared_prefix_and_zero_length_rows():
    import torch
    print("[gpu] int8 shared prefix, zero-length rows", flush=True)
    w = workloads.make_custom([1, 5, 20, 2, 3, 40, 7, 9], hq=8, hkv=2, d=128, dtype="bf16",
                              seed=8, prompt_lens=[21, 32, 45], prompt_of=[0, 0, 0, 1, 1, 1, 2, 2])
    _, _, _, ref = step.run_int8(w)
    db = runner.DeviceBatch(w, int8=True)
    db.prefill()
    db.step()
    assert_close(db.out_bits(), ref, "bf16", "int8 shared prefix")
    lens = db.context_lens.clone()
    db.context_lens[2] = 0
    db.decode()
    out = to_f64(db.out_bits(), "bf16")
    assert np.all(out[2] == 0)
    keep = [s for s in range(w.num_seqs) if s != 2]
    assert_close(db.out_bits()[keep], ref[keep], "bf16", "int8 other rows")
    db.context_lens.copy_(lens)


_FULL = {}


def _full(config):
    if config not in _FULL:
        _FULL.clear()
        import torch
        w = workloads.make(config)
        db = runner.DeviceBatch(w, int8=True)
        db.prefill()
        db.step()
        torch.cuda.synchronize()
        _FULL[config] = (w, db)
    return _FULL[config]


_ORACLE = {}


def _oracle_full(config):
    """The oracle's INT8 run of the same workload: (plan, k_codes, v_codes, out)."""
    if config not in _ORACLE:
        _ORACLE.clear()
        w, _ = _full(config)
        _ORACLE[config] = step.run_int8(w)
    return _ORACLE[config]


@pytest.mark.parametrize("config", [2, 3, 5])
def test_full_size_every_output_and_code_against_oracle(config):
    print(f"[gpu] int8 full-size workload {config}: every output and every code", flush=True)
    w, db = _full(config)
    _, k_ref, v_ref, ref = _oracle_full(config)
    info = assert_close(db.out_bits(), ref, w.dtype, f"int8 workload {config}")
    print(f"  {w.num_seqs} sequences x {w.num_q_heads} heads: {info}", flush=True)
    k, v = _codes(db)
    nb = w.num_blocks
    assert np.array_equal(k[:nb], k_ref) and np.array_equal(v[:nb], v_ref)


def test_full_size_split_equals_unsplit_and_is_deterministic():
    import torch
    print("[gpu] int8 full-size workload 3: split/unsplit/determinism", flush=True)
    w, db = _full(3)
    base = db.out_bits()
    out2 = torch.empty_like(db.out)
    db.decode(out=out2)
    assert np.array_equal(bits_of(out2), base)
    b = to_f64(base, w.dtype)
    ulp = 2.0 ** -7
    for ps in (pa.PARTITION_NONE, 256, 1024):
        db.decode(partition_size=ps, out=out2)
        c = to_f64(bits_of(out2), w.dtype)
        ratio = np.abs(c - b) / (ulp * np.abs(b) + 1e-5)
        assert ratio.max() <= 1.0, f"partition {ps}: {ratio.max():.2f} ulp"


@pytest.mark.parametrize("partition_size", [pa.PARTITION_AUTO, pa.PARTITION_NONE, 64])
def test_fused_step_equals_write_then_decode(partition_size):
    import torch
    print(f"[gpu] int8 fused step P={partition_size}", flush=True)
    w = workloads.make_custom([1, 5, 20, 2, 3, 40, 700, 9], hq=8, hkv=2, d=128, dtype="bf16",
                              seed=33, prompt_lens=[21, 32, 45],
                              prompt_of=[0, 0, 0, 1, 1, 1, 2, 2])
    a = runner.DeviceBatch(w, int8=True)
    b = runner.DeviceBatch(w, int8=True)
    for db, fused in ((a, True), (b, False)):
        db.prefill()
        db.step(partition_size=partition_size, fused=fused)
    torch.cuda.synchronize()
    for x, y in zip(a.caches[0], b.caches[0]):
        assert torch.equal(x, y)
    assert np.array_equal(a.out_bits(), b.out_bits())
    _, _, _, ref = step.run_int8(w)
    assert_close(a.out_bits(), ref, "bf16", "int8 fused step")
