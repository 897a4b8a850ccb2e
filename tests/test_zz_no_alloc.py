"""pa_paged_attention_decode_noalloc (workspace in the library's scratch array)
against pa_paged_attention_decode (caller's workspace): the same kernels, so
the outputs must be identical bit for bit -- on a full-size workload, then on
a smaller batch right after it (the scratch still holds the first call's
contents), and a call that needs more than the array is refused before any
launch.
"""
import ctypes

import numpy as np
import pytest

import paged_kv_cache_06_amd as pa
import workloads
from paged_kv_cache_06_amd import runner
from tests.helpers import bits_of

pytestmark = pytest.mark.gpu


def _both(db, partition_size):
    import torch
    kc, vc = db.caches[0]
    ref = torch.full_like(db.out, float("nan"))
    got = torch.full_like(db.out, float("nan"))
    pa.paged_attention_decode(db.q, kc, vc, db.tables, db.context_lens, db.w.scale, ref,
                              max_context_len=db.max_context_len, partition_size=partition_size)
    pa.paged_attention_decode_noalloc(db.q, kc, vc, db.tables, db.context_lens, db.w.scale, got,
                                      max_context_len=db.max_context_len,
                                      partition_size=partition_size)
    torch.cuda.synchronize()
    return bits_of(ref), bits_of(got)


def test_noalloc_equals_the_workspace_entry_point_on_two_calls_in_a_row():
    print("[gpu] no-alloc decode: full-size 70B-layer batch, then a small batch", flush=True)
    w = workloads.make(3)
    need = pa.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.head_dim,
                                     int(np.max(w.context_lens)), pa.PARTITION_AUTO)
    assert need <= pa.DECODE_SCRATCH_BYTES
    db = runner.DeviceBatch(w)
    db.prefill()
    db.step()
    ref, got = _both(db, pa.PARTITION_AUTO)
    assert np.array_equal(got, ref)
    assert np.array_equal(got, db.out_bits())
    # second call, smaller, split into many partials: stale scratch must not matter
    w2 = workloads.make_custom([1, 17, 300, 700, 2000], hq=16, hkv=2, d=64, dtype="f16", seed=77)
    db2 = runner.DeviceBatch(w2)
    db2.prefill()
    db2.step(partition_size=64)
    ref2, got2 = _both(db2, 64)
    assert np.array_equal(got2, ref2)
    assert np.all(np.isfinite(got2.view(np.float16)))


def test_noalloc_refuses_a_call_larger_than_its_scratch():
    import torch
    print("[gpu] no-alloc decode: oversize request refused", flush=True)
    # 4096 sequences x 64 heads x 32 partitions of partials need ~4 GiB: the
    # host check refuses the call before anything is launched or read
    s, hq, hkv, d, mcl, part = 4096, 64, 8, 128, 8192, 256
    assert pa.decode_workspace_bytes(s, hq, d, mcl, part) > pa.DECODE_SCRATCH_BYTES
    lib = pa.load()
    p = ctypes.c_void_p(256)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.pa_paged_attention_decode_noalloc(p, p, p, p, p, 1.0, p, s, hq, hkv, d, mcl // 16,
                                               mcl, part, 2, stream)
    assert st == -6  # PA_ERR_WORKSPACE
