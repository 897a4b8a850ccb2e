"""The C++ pool (through the C ABI) against the oracle pool, bit-exact, on the CPU."""
import random

import numpy as np
import pytest

import paged_kv_cache_06_amd as pa
import workloads
from oracle import pool as opool
from oracle import step
from paged_kv_cache_06_amd import runner


def test_random_operation_sequences_match_the_oracle():
    for seed in range(5):
        rnd = random.Random(seed)
        nb = rnd.choice([8, 64, 200])
        order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
        ref = opool.BlockPool(nb, order)
        lib = pa.Pool(nb, order)
        cap = 40
        tabs_ref, tabs_lib, lens = [], [], []
        for _ in range(1500):
            op = rnd.random()
            if op < 0.5 and lens:
                i = rnd.randrange(len(lens))
                n = rnd.randint(0, 40)
                err_ref = err_lib = None
                try:
                    out_ref = ref.append(tabs_ref[i], lens[i], n, max_blocks=cap)
                except opool.PoolError as e:
                    err_ref = type(e).__name__
                row, nb_ = tabs_lib[i]
                try:
                    slots, nb2, cow = lib.append_slots(row, nb_, lens[i], n)
                except pa.PAError as e:
                    err_lib = {-1: "InvalidArg", -2: "OutOfBlocks", -3: "BadBlock"}[e.status]
                assert err_ref == err_lib
                if err_ref is None:
                    assert list(slots) == out_ref[0] and cow == out_ref[1]
                    tabs_lib[i] = (row, nb2)
                    lens[i] += n
            elif op < 0.62 and lens:
                i = rnd.randrange(len(lens))
                tabs_ref.append(ref.fork(tabs_ref[i]))
                row, nb_ = tabs_lib[i]
                lib.fork(row[:nb_])
                tabs_lib.append((row.copy(), nb_))
                lens.append(lens[i])
            elif op < 0.8 and lens:
                i = rnd.randrange(len(lens))
                ref.free_table(tabs_ref.pop(i))
                row, nb_ = tabs_lib.pop(i)
                lib.free_table(row[:nb_])
                lens.pop(i)
            else:
                tabs_ref.append([])
                tabs_lib.append((np.zeros(cap, np.int32), 0))
                lens.append(0)
            for (row, nb_), t in zip(tabs_lib, tabs_ref):
                assert row[:nb_].tolist() == t
            assert [lib.refcount(b) for b in range(nb)] == ref.refcount
            assert lib.num_free() == ref.num_free()
        st = lib.stats()
        assert st["copies"] == ref.copies_made and st["free"] == ref.num_free()


def test_single_block_calls_and_errors_match():
    ref = opool.BlockPool(3, [2, 0, 1])
    lib = pa.Pool(3, [2, 0, 1])
    assert [lib.alloc() for _ in range(3)] == [ref.alloc() for _ in range(3)] == [2, 0, 1]
    with pytest.raises(pa.OutOfBlocks):
        lib.alloc()
    lib.free(0)
    ref.free(0)
    assert lib.alloc() == ref.alloc() == 0
    lib.incref(1)
    with pytest.raises(pa.PAError) as e:
        lib.free(7)
    assert e.value.status == -3
    lib.free(1)
    lib.free(1)
    with pytest.raises(pa.PAError):
        lib.free(1)  # double free
    with pytest.raises(pa.PAError):
        lib.incref(1)
    with pytest.raises(pa.PAError):
        lib.fork([2, 1])  # all-or-nothing: 1 is not held
    assert lib.refcount(2) == 1
    assert lib.refcount(99) == -1


@pytest.mark.parametrize("config", [1, 2, 3, 4, "4b", 5])
def test_workload_tables_slots_and_copies_match_the_oracle(config):
    w = workloads.make(config, values=False)
    ref = step.plan(w)
    bm, phases = runner.plan(w)
    for s in range(w.num_seqs):
        assert bm.table(s) == ref.tables[s]
    # table padding points at the extra poison block
    for s in range(w.num_seqs):
        assert np.all(bm.rows[s, len(ref.tables[s]):] == w.num_blocks)
    for ph_lib, ph_ref in zip(phases, ref.phases):
        assert np.array_equal(ph_lib.pairs, ph_ref.pairs)
        assert np.array_equal(ph_lib.slots, ph_ref.slots)
    assert [bm.pool.refcount(b) for b in range(w.num_blocks)] == ref.pool.refcount
    assert bm.pool.num_free() == ref.pool.num_free()
    if config == 4:
        assert len(phases[2].pairs) == 192


def test_workload_token_values_follow_the_same_slots():
    w = workloads.make_custom([1, 5, 20, 2, 3, 40], hq=4, hkv=2, d=8, dtype="bf16", seed=8,
                              prompt_lens=[21, 32], prompt_of=[0, 0, 0, 1, 1, 1])
    ref = step.plan(w)
    _, phases = runner.plan(w)
    for a, b in zip(phases, ref.phases):
        assert np.array_equal(a.key, b.key) and np.array_equal(a.value, b.value)
