"""Pins of the host tier: oracle.pool.swap_blocks and oracle.cache_ops.transfer_blocks."""
import random

import numpy as np
import pytest

import workloads
from oracle import attention, cache_ops, step
from oracle.pool import BadBlock, BlockPool, OutOfBlocks, blocks_for, swap_blocks


def _conservation(pool, tables):
    counts = [0] * pool.num_blocks
    for t in tables:
        for b in t:
            counts[b] += 1
    assert counts == pool.refcount
    assert pool.num_free() + sum(1 for c in counts if c > 0) == pool.num_blocks


def test_swap_out_and_back_in_restores_every_sequence_exactly():
    """Swap every sequence of a shared-prefix batch out to a host pool and back
    into the device pool: the device tables change, each sequence's gathered
    K/V bits and its decode output do not."""
    w = workloads.make_custom([1, 5, 20, 2, 3, 40, 7, 9], hq=8, hkv=2, d=16, dtype="bf16",
                              seed=5, prompt_lens=[21, 32, 45], prompt_of=[0, 0, 0, 1, 1, 1, 2, 2])
    pl, kc, vc, want = step.run(w, np.uint16(0x7FC0))
    gpu = pl.pool
    tables = [list(t) for t in pl.tables]
    cpu = BlockPool(200, free_order=random.Random(1).sample(range(200), 200))
    hk = np.zeros((200,) + kc.shape[1:], kc.dtype)
    hv = np.zeros_like(hk)
    host_tables = []
    for t in tables:
        pairs = swap_blocks(gpu, cpu, t)
        cache_ops.transfer_blocks(kc, vc, hk, hv, pairs)
        host_tables.append([d for _, d in pairs])
    assert gpu.num_free() == gpu.num_blocks  # every device reference moved
    _conservation(cpu, host_tables)
    kc[:] = np.uint16(0x7FC0)  # the device copies are gone
    vc[:] = np.uint16(0x7FC0)
    back = []
    for t in host_tables:
        pairs = swap_blocks(cpu, gpu, t)
        cache_ops.transfer_blocks(hk, hv, kc, vc, pairs)
        back.append([d for _, d in pairs])
    assert cpu.num_free() == cpu.num_blocks
    _conservation(gpu, back)
    assert back != tables  # new physical blocks ...
    width = max(len(t) for t in back)
    tab = np.zeros((len(back), width), np.int64)
    for s, t in enumerate(back):
        tab[s, :len(t)] = t
    got = attention.paged_decode(w.q, kc, vc, tab, pl.context_lens, w.scale, w.dtype)
    assert np.array_equal(got, want)  # ... the same attention, bit for bit


def test_a_shared_block_stays_for_the_other_sharers():
    gpu = BlockPool(8, free_order=range(8))
    cpu = BlockPool(8, free_order=range(8))
    a = []
    gpu.append(a, 0, 20)  # blocks 0, 1
    b = gpu.fork(a)
    pairs = swap_blocks(gpu, cpu, b)
    assert pairs == [(0, 0), (1, 1)]
    assert gpu.refcount[0] == gpu.refcount[1] == 1  # still held by a
    assert gpu.num_free() == 6
    _conservation(gpu, [a])
    _conservation(cpu, [[0, 1]])


def test_swap_is_all_or_nothing():
    gpu = BlockPool(8)
    cpu = BlockPool(2)
    t = []
    gpu.append(t, 0, 48)  # 3 blocks
    before = (list(gpu.refcount), list(gpu.free_stack), list(cpu.refcount), list(cpu.free_stack))
    with pytest.raises(OutOfBlocks):
        swap_blocks(gpu, cpu, t)
    with pytest.raises(BadBlock):
        swap_blocks(gpu, cpu, [t[0], 7])  # block 7 is not held
    assert (list(gpu.refcount), list(gpu.free_stack), list(cpu.refcount),
            list(cpu.free_stack)) == before


def _snapshot(*pools):
    return [(list(p.refcount), list(p.free_stack)) for p in pools]


def test_a_block_listed_more_often_than_held_changes_nothing():
    """Each listing of a block moves one reference the caller holds, and a
    swap is all or nothing ("KV Cache and PagedAttention: why your LLM server
    slows down", section "How PagedAttention fixes this": single pages move to
    the CPU; reading R18): a block held once and listed twice is refused with
    both pools' counts and free stacks exactly as they were."""
    gpu = BlockPool(8, free_order=range(8))
    cpu = BlockPool(8, free_order=range(8))
    t = []
    gpu.append(t, 0, 32)  # blocks 0 and 1, one reference each
    before = _snapshot(gpu, cpu)
    with pytest.raises(BadBlock):
        swap_blocks(gpu, cpu, [t[0], t[1], t[0]])
    assert _snapshot(gpu, cpu) == before
    with pytest.raises(BadBlock):
        swap_blocks(gpu, cpu, [t[1], t[1]])
    assert _snapshot(gpu, cpu) == before


def test_a_block_held_twice_and_listed_twice_moves_both_references():
    """Two holders of one block (a fork) swapping it together: each listing
    gets its own destination block and drops one source reference, so the
    source block is free afterwards and each copy is held once."""
    gpu = BlockPool(8, free_order=range(8))
    cpu = BlockPool(8, free_order=range(8))
    a = []
    gpu.append(a, 0, 16)  # block 0
    gpu.fork(a)           # a second holder: count 2
    pairs = swap_blocks(gpu, cpu, [a[0], a[0]])
    assert pairs == [(0, 0), (0, 1)]
    assert gpu.refcount[0] == 0 and gpu.num_free() == 8
    assert cpu.refcount[0] == cpu.refcount[1] == 1 and cpu.num_free() == 6


def test_fine_grained_eviction_moves_only_what_is_needed():
    """The page's contrast: freeing k device blocks by moving single blocks
    moves k of them; moving whole sequences moves every block of each
    sequence it has to take."""
    lens = [40 * 16, 40 * 16, 40 * 16]  # three sequences of 40 blocks
    for k in (1, 5, 39, 41):
        gpu = BlockPool(120)
        tables = []
        for n in lens:
            t = []
            gpu.append(t, 0, n)
            tables.append(t)
        fine_cpu, whole_cpu = BlockPool(200), BlockPool(200)
        # fine-grained: the last k blocks of the latest sequences
        victims = []
        for t in reversed(tables):
            victims += t[::-1][:k - len(victims)]
            if len(victims) == k:
                break
        g1 = BlockPool(120)
        for n in lens:
            g1.append([], 0, n)
        moved_fine = len(swap_blocks(g1, fine_cpu, victims))
        # whole sequences, latest first, until k blocks are free
        g2 = BlockPool(120)
        t2 = []
        for n in lens:
            t = []
            g2.append(t, 0, n)
            t2.append(t)
        moved_whole = 0
        while g2.num_free() < k:
            moved_whole += len(swap_blocks(g2, whole_cpu, t2.pop()))
        assert moved_fine == k == g1.num_free()
        assert moved_whole == 40 * blocks_for(k * 16, 40 * 16)


def test_random_swaps_conserve_references_in_both_tiers():
    rnd = random.Random(9)
    gpu, cpu = BlockPool(40), BlockPool(40)
    seqs = []  # (tier, table)
    for _ in range(2000):
        op = rnd.random()
        try:
            if op < 0.3:
                t = []
                gpu.append(t, 0, rnd.randint(1, 80))
                seqs.append(["gpu", t])
            elif op < 0.45 and seqs:
                sq = rnd.choice(seqs)
                if sq[0] == "gpu":
                    seqs.append(["gpu", gpu.fork(sq[1])])
            elif op < 0.75 and seqs:
                sq = rnd.choice(seqs)
                src, dst = (gpu, cpu) if sq[0] == "gpu" else (cpu, gpu)
                pairs = swap_blocks(src, dst, sq[1])
                sq[0] = "cpu" if sq[0] == "gpu" else "gpu"
                sq[1] = [d for _, d in pairs]
            elif seqs:
                tier, t = seqs.pop(rnd.randrange(len(seqs)))
                (gpu if tier == "gpu" else cpu).free_table(t)
        except OutOfBlocks:
            pass
        _conservation(gpu, [t for tier, t in seqs if tier == "gpu"])
        _conservation(cpu, [t for tier, t in seqs if tier == "cpu"])
