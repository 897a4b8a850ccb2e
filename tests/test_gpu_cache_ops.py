"""reshape_and_cache and copy_blocks on the GPU, bit-exact against the oracle."""
import numpy as np
import pytest

import paged_kv_cache_06_amd as pa
import workloads
from oracle import cache_ops, step
from paged_kv_cache_06_amd import runner
from tests.helpers import NAN_BITS, bits_of

pytestmark = pytest.mark.gpu


def _device_logical(db):
    out = []
    for kc, vc in db.caches:
        k, v = pa.logical_view(kc, vc)
        out.append((bits_of(k), bits_of(v)))
    return out


def _same_bits(a, b):
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("f16", 128), ("bf16", 64),
                                     ("f32", 32), ("f16", 256)])
def test_prefill_and_step_writes_match_oracle_bits(dtype, d):
    print(f"[gpu] cache writes dtype={dtype} d={d}", flush=True)
    w = workloads.make_custom([1, 15, 16, 17, 40, 130], hq=4, hkv=2, d=d, dtype=dtype, seed=21)
    ref = step.plan(w)
    kc_ref, vc_ref = step.empty_cache(w, NAN_BITS[dtype])
    for ph in ref.phases:
        step.apply_phase(ph, kc_ref, vc_ref)
    db = runner.DeviceBatch(w)
    db.prefill()
    db.step()
    import torch
    torch.cuda.synchronize()
    (k, v), = _device_logical(db)
    assert _same_bits(k[:w.num_blocks], kc_ref) and _same_bits(v[:w.num_blocks], vc_ref)
    # the poison block is untouched
    assert _same_bits(k[w.num_blocks:], np.full_like(k[w.num_blocks:], NAN_BITS[dtype]))


def test_copy_on_write_step_matches_oracle_bits():
    print("[gpu] copy-on-write step", flush=True)
    w = workloads.make_custom([1, 5, 20, 2, 3, 40, 7, 9], hq=8, hkv=2, d=128, dtype="bf16",
                              seed=8, prompt_lens=[21, 32, 45], prompt_of=[0, 0, 0, 1, 1, 1, 2, 2])
    ref = step.plan(w)
    assert len(ref.phases[2].pairs) == 3
    kc_ref, vc_ref = step.empty_cache(w, NAN_BITS["bf16"])
    for ph in ref.phases:
        step.apply_phase(ph, kc_ref, vc_ref)
    db = runner.DeviceBatch(w)
    db.prefill()
    db.step()
    (k, v), = _device_logical(db)
    assert _same_bits(k[:w.num_blocks], kc_ref) and _same_bits(v[:w.num_blocks], vc_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_copy_blocks_random_pairs_and_skips(dtype):
    import torch
    print(f"[gpu] copy_blocks random dtype={dtype}", flush=True)
    rng = np.random.default_rng(3)
    nb, hkv, d = 40, 4, 64
    w = workloads.make_custom([nb * 16], hq=4, hkv=hkv, d=d, dtype=dtype, seed=4,
                              num_blocks=nb)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    kc, vc = pa.new_kv_cache(nb, hkv, d, tdt, "cuda")
    # fill every slot with the workload's tokens (slot = token index)
    kdev, vdev = runner.to_device(w.k_private, dtype), runner.to_device(w.v_private, dtype)
    slots = torch.arange(nb * 16, dtype=torch.int64, device="cuda")
    pa.reshape_and_cache(kdev, vdev, kc, vc, slots)
    k0, v0 = (bits_of(x) for x in pa.logical_view(kc, vc))
    src = rng.choice(20, size=10, replace=False)
    dst = 20 + rng.choice(20, size=10, replace=False)
    pairs = np.stack([src, dst], 1).astype(np.int64)
    pairs = np.concatenate([pairs, [[-1, 5], [3, nb], [nb + 7, 2]]])  # invalid pairs: skipped
    pa.copy_blocks(kc, vc, torch.from_numpy(pairs).cuda())
    k1, v1 = (bits_of(x) for x in pa.logical_view(kc, vc))
    kr, vr = k0.copy(), v0.copy()
    cache_ops.copy_blocks(kr, vr, pairs[:10])
    assert _same_bits(k1, kr) and _same_bits(v1, vr)


def _run(blocks, start_row, n):
    """Slots of n consecutive positions from row start_row of blocks[0] on."""
    return [int(blocks[(start_row + i) // 16]) * 16 + (start_row + i) % 16 for i in range(n)]


@pytest.mark.parametrize("dtype,hkv,d", [("bf16", 8, 128), ("f16", 2, 64), ("bf16", 1, 256)])
def test_token_runs_match_oracle_bits(dtype, hkv, d):
    """Runs of new tokens through the windowed writer: aligned runs over whole
    blocks, groups holding a skipped and an out-of-range slot, a run that
    starts mid-block and crosses into another block, scattered slots and a
    partial last window, bit for bit against the oracle."""
    import torch
    print(f"[gpu] token runs {dtype} hkv={hkv} d={d}", flush=True)
    nb = 40
    rng = np.random.default_rng(hkv * d)
    perm = rng.permutation(nb)
    group = _run(perm[5:6], 0, 16)
    group[3], group[12] = -1, nb * 16 + 100   # skipped, out of range
    scattered = rng.choice(np.arange(6 * 16, 16 * 16), 25, replace=False)
    slots = (_run(perm[0:2], 0, 32) + group + _run(perm[4:5], 8, 8) + _run(perm[2:4], 5, 20)
             + [int(perm[b // 16]) * 16 + b % 16 for b in scattered] + _run(perm[16:17], 0, 7))
    slots = np.asarray(slots, np.int64)
    T = len(slots)
    valid = (slots >= 0) & (slots < nb * 16)
    assert len(set(slots[valid].tolist())) == valid.sum()  # no slot written twice
    pieces = [q for q in range(0, T - 7, 8)
              if valid[q:q + 8].all() and slots[q] % 8 == 0
              and (slots[q:q + 8] == slots[q] + np.arange(8)).all()]
    assert pieces == [0, 8, 16, 24, 48]  # aligned groups of 8; the rest are not
    bits = {"bf16": np.uint16, "f16": np.uint16}[dtype]
    key = rng.integers(0, 0x7B00, (T, hkv, d)).astype(bits)   # finite values
    value = rng.integers(0, 0x7B00, (T, hkv, d)).astype(bits)
    kc_ref = np.full((nb, hkv, 16, d), NAN_BITS[dtype], bits)
    vc_ref = kc_ref.copy()
    cache_ops.reshape_and_cache(key, value, kc_ref, vc_ref, np.where(valid, slots, -1))
    kc, vc = pa.new_kv_cache(nb, hkv, d, runner.torch_dtype(dtype), "cuda", float("nan"))
    pa.reshape_and_cache(runner.to_device(key, dtype), runner.to_device(value, dtype), kc, vc,
                         torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    k, v = pa.logical_view(kc, vc)
    assert _same_bits(bits_of(k), kc_ref) and _same_bits(bits_of(v), vc_ref)


def test_slot_minus_one_and_out_of_range_are_skipped():
    import torch
    print("[gpu] skipped slots", flush=True)
    kc, vc = pa.new_kv_cache(4, 2, 64, torch.float16, "cuda", fill=0.0)
    key = torch.ones(3, 2, 64, dtype=torch.float16, device="cuda")
    slots = torch.tensor([-1, 4 * 16, 17], dtype=torch.int64, device="cuda")
    pa.reshape_and_cache(key, key * 2, kc, vc, slots)
    k, v = pa.logical_view(kc, vc)
    k, v = k.cpu().float(), v.cpu().float()
    assert k[1, :, 1].eq(1).all() and v[1, :, 1].eq(2).all()
    assert k.sum().item() == 2 * 64 and v.sum().item() == 2 * 2 * 64


@pytest.mark.parametrize("config", [2, 3, 4, 5])
def test_full_size_cache_after_the_step_matches_oracle_bits(config):
    """At full size, in the benchmark's step: every block of both caches after
    the prefill and the step (copy-on-write copies, then the step's token
    writes) equals the oracle's cache bit for bit -- written slots, copied
    blocks and never-written (NaN) slots alike -- and every copy-on-write copy
    holds its source's pre-step contents outside the slots the step wrote."""
    import torch
    print(f"[gpu] full-size cache after the step, workload {config}", flush=True)
    w = workloads.make(config)
    ref = step.plan(w)
    kc_ref, vc_ref = step.empty_cache(w, NAN_BITS[w.dtype])
    for ph in ref.phases:
        step.apply_phase(ph, kc_ref, vc_ref)
    db = runner.DeviceBatch(w)
    db.prefill()
    torch.cuda.synchronize()
    B = db.phases[2]
    assert np.array_equal(B.pairs, ref.phases[2].pairs)
    kc, vc = db.caches[0]
    before = {}
    for src, dst in B.pairs.tolist():
        kb, vb = pa.logical_view(kc[src:src + 1], vc[src:src + 1])
        before[dst] = (bits_of(kb)[0], bits_of(vb)[0])
    db.step()
    torch.cuda.synchronize()
    (k, v), = _device_logical(db)
    nb = w.num_blocks
    assert _same_bits(k[:nb], kc_ref) and _same_bits(v[:nb], vc_ref)
    assert _same_bits(k[nb:], np.full_like(k[nb:], NAN_BITS[w.dtype]))  # poison block
    written = set(B.slots.tolist())
    for dst, (kb, vb) in before.items():
        keep = [r for r in range(16) if dst * 16 + r not in written]
        assert np.array_equal(k[dst][:, keep], kb[:, keep])
        assert np.array_equal(v[dst][:, keep], vb[:, keep])
    print(f"  {nb} blocks, {len(B.slots)} step tokens, {len(B.pairs)} copies", flush=True)
    if config == 4:
        assert len(B.pairs) == 192  # 64 prompts x (4 - 1) writers of the shared partial block
