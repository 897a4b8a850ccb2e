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


@pytest.mark.parametrize("config", [2, 4])
def test_full_size_step_writes(config):
    """At full size: the step's tokens land in their slots, and (shared prefix) every
    copy holds the source block's pre-step contents outside the written slots."""
    import torch
    print(f"[gpu] full-size step writes config={config}", flush=True)
    w = workloads.make(config)
    db = runner.DeviceBatch(w)
    db.prefill()
    torch.cuda.synchronize()
    B = db.phases[2]
    kc, vc = db.caches[0]
    before = {}
    for src, dst in B.pairs[:16].tolist():
        kb, vb = pa.logical_view(kc[src:src + 1], vc[src:src + 1])
        before[dst] = (bits_of(kb)[0], bits_of(vb)[0])
    db.step()
    torch.cuda.synchronize()
    k, v = (bits_of(x) for x in pa.logical_view(kc, vc))
    sl = B.slots
    assert np.array_equal(k[sl // 16, :, sl % 16, :], B.key)
    assert np.array_equal(v[sl // 16, :, sl % 16, :], B.value)
    written = set(sl.tolist())
    for dst, (kb, vb) in before.items():
        for r in range(16):
            if dst * 16 + r not in written:
                assert np.array_equal(k[dst, :, r], kb[:, r])
                assert np.array_equal(v[dst, :, r], vb[:, r])
