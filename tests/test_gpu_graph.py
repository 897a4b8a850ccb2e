"""Graph capture of the hot path: a decode step (cache writes + plan + decode
with in-kernel merges; bf16 and INT8 caches; with copy-on-write block copies)
and a chunked prefill, captured once in a HIP graph through torch and
replayed several times with other eager work and a NaN overwrite of the
output in between.  Every replay must equal the eager result bit for bit
(the library's launches record no memset, allocation or synchronisation)."""
import numpy as np
import pytest

import workloads
from paged_kv_cache_06_amd import runner
from tests.helpers import bits_of

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _eager_noise(torch, db):
    # unrelated eager work on the same stream, then a different decode of the
    # same batch into a scratch output (another partition size, own workspace)
    x = torch.randn(1 << 20, device="cuda")
    (x * 2).sum().item()
    scratch = torch.empty_like(db.out)
    db.decode(partition_size=0, out=scratch)


def _capture(torch, fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up off the default stream (workspaces exist before capture)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("int8", [False, True])
def test_decode_step_graph_replays_match_eager(int8):
    import torch
    print(f"[gpu] decode step in a graph, int8={int8}", flush=True)
    w = workloads.make_custom([1, 17, 300, 1500, 5000, 40], hq=16, hkv=2, d=128, dtype="bf16",
                              seed=31)
    db = runner.DeviceBatch(w, int8=int8)
    db.prefill()
    db.step(partition_size=512)  # splits: the in-kernel merge runs
    torch.cuda.synchronize()
    ref = bits_of(db.out)
    g = _capture(torch, lambda: db.step(partition_size=512))
    for r in range(REPLAYS):
        db.out.fill_(float("nan"))
        _eager_noise(torch, db)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(db.out), ref), f"replay {r}"


def test_decode_step_with_block_copies_graph_replays_match_eager():
    import torch
    print("[gpu] decode step with copy-on-write copies in a graph", flush=True)
    w = workloads.make_custom([5, 20, 1, 33], hq=8, hkv=2, d=64, dtype="bf16", seed=32,
                              prompt_lens=[100, 40], prompt_of=[0, 0, 1, 1])
    db = runner.DeviceBatch(w)
    assert db.dev_phases[2]["pairs"].shape[0] > 0
    db.prefill()
    db.step()
    torch.cuda.synchronize()
    ref = bits_of(db.out)
    g = _capture(torch, db.step)
    for r in range(REPLAYS):
        db.out.fill_(float("nan"))
        _eager_noise(torch, db)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(db.out), ref), f"replay {r}"


def test_prefill_graph_replays_match_eager():
    import torch
    print("[gpu] chunked prefill in a graph", flush=True)
    w = workloads.make_prefill([33, 64, 7, 90], [200, 0, 1000, 45], hq=32, hkv=8, d=128,
                               dtype="bf16", seed=33)
    db = runner.DeviceBatch(w)
    db.prefill()
    db._apply(db.dev_phases[2], db.caches[0])
    ref = bits_of(db.attend_chunks())
    torch.cuda.synchronize()
    g = _capture(torch, db.attend_chunks)
    for r in range(REPLAYS):
        db.chunk_out.fill_(float("nan"))
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(db.chunk_out), ref), f"replay {r}"
