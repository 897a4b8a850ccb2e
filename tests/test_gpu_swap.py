"""Moving blocks between the device cache and a pinned host cache (the host
tier) on the GPU: bit-exact against the oracle's block copies, and a batch
swapped out and back in decodes bit-identically."""
import numpy as np
import pytest

import paged_kv_cache_06_amd as pa
import workloads
from oracle import cache_ops
from paged_kv_cache_06_amd import runner

pytestmark = pytest.mark.gpu


def _np(t):
    import torch
    t = t.cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    return t.numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32", "i8"])
def test_transfer_round_trip_is_bit_exact(dtype):
    import torch
    print(f"[gpu] transfer blocks {dtype}", flush=True)
    nb, hkv, d = 40, 2, 128
    g = torch.Generator().manual_seed(3)
    if dtype == "i8":
        kd, vd = pa.new_kv_cache_int8(nb, hkv, d, "cuda")
        kd.copy_(torch.randint(-127, 128, kd.shape, generator=g, dtype=torch.int8))
        vd.copy_(torch.randint(-127, 128, vd.shape, generator=g, dtype=torch.int8))
        kh, vh = pa.new_host_kv_cache(30, hkv, d, torch.int8)
    else:
        tdt = runner.torch_dtype(dtype)
        kd, vd = pa.new_kv_cache(nb, hkv, d, tdt, "cuda")
        kd.copy_(torch.randn(kd.shape, generator=g).to(tdt))
        vd.copy_(torch.randn(vd.shape, generator=g).to(tdt))
        kh, vh = pa.new_host_kv_cache(30, hkv, d, tdt)
    kh.zero_()
    vh.zero_()
    pairs = np.array([[5, 0], [39, 29], [0, 7], [17, 3], [41, 4], [6, -1]], np.int64)  # 2 skipped
    pd = torch.from_numpy(pairs).cuda()
    ref_k, ref_v = _np(kh).copy(), _np(vh).copy()
    cache_ops.transfer_blocks(_np(kd), _np(vd), ref_k, ref_v, pairs[:4])
    pa.transfer_blocks(kd, vd, kh, vh, pd)  # device -> host, pairs on the device
    torch.cuda.synchronize()
    assert np.array_equal(_np(kh), ref_k) and np.array_equal(_np(vh), ref_v)
    back = np.array([[0, 1], [29, 2], [7, 8], [3, 9]], np.int64)
    kd2, vd2 = torch.zeros_like(kd), torch.zeros_like(vd)
    pa.transfer_blocks(kh, vh, kd2, vd2, torch.from_numpy(back).pin_memory())  # pinned pairs
    torch.cuda.synchronize()
    want_k, want_v = np.zeros_like(_np(kd)), np.zeros_like(_np(vd))
    cache_ops.transfer_blocks(ref_k, ref_v, want_k, want_v, back)
    assert np.array_equal(_np(kd2), want_k) and np.array_equal(_np(vd2), want_v)
    assert pa.release_finished_transfers() == 0  # both copies done: no host tensor held


def test_pageable_host_memory_is_refused():
    import torch
    print("[gpu] transfer refuses pageable memory", flush=True)
    kd, vd = pa.new_kv_cache(8, 2, 64, torch.bfloat16, "cuda", 0.0)
    kh = torch.zeros(kd.shape, dtype=torch.bfloat16)  # not pinned
    vh = torch.zeros(vd.shape, dtype=torch.bfloat16)
    pairs = torch.tensor([[0, 0]], dtype=torch.int64, device="cuda")
    lib = pa.load()
    import ctypes
    st = lib.pa_transfer_blocks(ctypes.c_void_p(kd.data_ptr()), ctypes.c_void_p(vd.data_ptr()), 8,
                                ctypes.c_void_p(kh.data_ptr()), ctypes.c_void_p(vh.data_ptr()), 8,
                                ctypes.c_void_p(pairs.data_ptr()), 1, 2, 64, 2, None)
    assert st == -1


@pytest.mark.parametrize("int8", [False, True])
def test_batch_swapped_out_and_back_in_decodes_identically(int8):
    import torch
    print(f"[gpu] swap a batch out and back in (int8={int8})", flush=True)
    w = workloads.make_custom([1, 5, 20, 2, 3, 40, 7, 9], hq=8, hkv=2, d=128, dtype="bf16",
                              seed=8, prompt_lens=[21, 32, 45], prompt_of=[0, 0, 0, 1, 1, 1, 2, 2])
    db = runner.DeviceBatch(w, int8=int8)
    db.prefill()
    db.step()
    torch.cuda.synchronize()
    base = db.out_bits().copy()
    kd, vd = db.caches[0]
    host = pa.Pool(64)
    kh, vh = pa.new_host_kv_cache(64, w.num_kv_heads, w.head_dim, kd.dtype)
    host_rows = []
    for s in range(w.num_seqs):
        nb = int(db.bm.nblocks[s])
        pairs = pa.swap_blocks(db.bm.pool, host, db.bm.rows[s, :nb])
        pa.transfer_blocks(kd, vd, kh, vh, torch.from_numpy(pairs).cuda())
        host_rows.append(pairs[:, 1].copy())
    torch.cuda.synchronize()
    assert db.bm.pool.num_free() == w.num_blocks  # the device pool is empty
    kd.fill_(127 if int8 else float("nan"))
    vd.fill_(127 if int8 else float("nan"))
    for s in range(w.num_seqs):
        pairs = pa.swap_blocks(host, db.bm.pool, host_rows[s])
        pa.transfer_blocks(kh, vh, kd, vd, torch.from_numpy(pairs).pin_memory())
        db.bm.rows[s, :len(pairs)] = pairs[:, 1]
    assert host.num_free() == 64
    db.tables.copy_(torch.from_numpy(db.bm.rows))
    db.decode()
    torch.cuda.synchronize()
    assert np.array_equal(db.out_bits(), base)
