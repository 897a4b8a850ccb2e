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


@pytest.mark.parametrize("config,prefix_cache", [(1, False), (2, False), (3, False), (4, False),
                                                 ("4b", False), (5, False), (4, True),
                                                 ("4b", True)])
def test_workload_tables_slots_and_copies_match_the_oracle(config, prefix_cache):
    w = workloads.make(config, values=False)
    ref = step.plan(w, prefix_cache)
    bm, phases = runner.plan(w, prefix_cache)
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
    if config == 4 and not prefix_cache:
        assert len(phases[2].pairs) == 192
    if prefix_cache:  # no shared partial block, so nothing to copy
        assert all(len(ph.pairs) == 0 for ph in phases)
        st = bm.pool.stats()
        assert st["cached"] == ref.pool.stats()["cached"] and st["prefix_hits"] == ref.pool.prefix_hits


def test_workload_token_values_follow_the_same_slots():
    w = workloads.make_custom([1, 5, 20, 2, 3, 40], hq=4, hkv=2, d=8, dtype="bf16", seed=8,
                              prompt_lens=[21, 32], prompt_of=[0, 0, 0, 1, 1, 1])
    ref = step.plan(w)
    _, phases = runner.plan(w)
    for a, b in zip(phases, ref.phases):
        assert np.array_equal(a.key, b.key) and np.array_equal(a.value, b.value)


def _err(fn):
    try:
        return fn(), None
    except opool.PoolError as e:
        return None, type(e).__name__
    except pa.PAError as e:
        return None, {-1: "InvalidArg", -2: "OutOfBlocks", -3: "BadBlock"}[e.status]


def test_prefix_cache_operation_sequences_match_the_oracle():
    """match / append / register / free / fork through the prefix cache, with
    token lists built from a few shared 16-token phrases so that prefixes
    repeat; tables, counts, free and cached totals, hits and errors must agree
    after every operation."""
    for seed in range(4):
        rnd = random.Random(100 + seed)
        nb = rnd.choice([12, 40, 96])
        order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
        ref = opool.BlockPool(nb, order)
        lib = pa.Pool(nb, order)
        cap = 12
        phrases = [[rnd.randrange(3) for _ in range(16)] for _ in range(3)]
        seqs = []  # [ref table, lib row, lib nblocks, tokens]
        for _ in range(1500):
            op = rnd.random()
            if op < 0.3:
                toks = sum((rnd.choice(phrases) for _ in range(rnd.randint(0, 4))), [])
                toks += [rnd.randrange(3) for _ in range(rnd.randint(0, 24))]
                if not toks:
                    continue
                t_ref = ref.match_prefix(toks)
                m_lib = lib.prefix_match(toks, cap)
                assert m_lib.tolist() == t_ref
                row = np.zeros(cap, np.int32)
                row[:len(m_lib)] = m_lib
                pos = 16 * len(t_ref)
                out_ref, e_ref = _err(lambda: ref.append(t_ref, pos, len(toks) - pos, max_blocks=cap))
                out_lib, e_lib = _err(lambda: lib.append_slots(row, len(m_lib), pos, len(toks) - pos))
                assert e_ref == e_lib
                if e_ref is not None:  # give the matched blocks back
                    ref.free_table(t_ref)
                    lib.free_table(m_lib)
                    continue
                assert list(out_lib[0]) == out_ref[0] and out_lib[2] is None and out_ref[1] is None
                seqs.append([t_ref, row, out_lib[1], toks])
                assert ref.register(t_ref, toks) == lib.prefix_register(row[:out_lib[1]], toks)
            elif op < 0.55 and seqs:
                sq = rnd.choice(seqs)
                t_ref, row, nbl, toks = sq
                new = rnd.choice([[rnd.randrange(3) for _ in range(rnd.randint(1, 20))],
                                  list(rnd.choice(phrases))])
                out_ref, e_ref = _err(lambda: ref.append(t_ref, len(toks), len(new), max_blocks=cap))
                out_lib, e_lib = _err(lambda: lib.append_slots(row, nbl, len(toks), len(new)))
                assert e_ref == e_lib
                if e_ref is None:
                    assert list(out_lib[0]) == out_ref[0] and out_lib[2] == out_ref[1]
                    sq[2] = out_lib[1]
                    toks.extend(new)
                    if out_ref[1] is None:  # a copied block would hold its source's tokens too
                        assert ref.register(t_ref, toks) == lib.prefix_register(row[:sq[2]], toks)
            elif op < 0.65 and seqs:
                sq = rnd.choice(seqs)
                seqs.append([ref.fork(sq[0]), sq[1].copy(), sq[2], list(sq[3])])
                lib.fork(sq[1][:sq[2]])
            elif op < 0.68 and seqs:
                sq = rnd.choice(seqs)
                bad = list(sq[3])
                if len(bad) >= 16:
                    bad[0] += 1  # claims other tokens for a (maybe cached) block
                    _, e_ref = _err(lambda: ref.register(sq[0], bad))
                    _, e_lib = _err(lambda: lib.prefix_register(sq[1][:sq[2]], bad))
                    assert e_ref == e_lib
            elif seqs:
                t_ref, row, nbl, _ = seqs.pop(rnd.randrange(len(seqs)))
                ref.free_table(t_ref)
                lib.free_table(row[:nbl])
            for t_ref, row, nbl, _ in seqs:
                assert row[:nbl].tolist() == t_ref
            assert [lib.refcount(b) for b in range(nb)] == ref.refcount
            st, so = lib.stats(), ref.stats()
            for k in ("free", "used", "shared", "copies", "cached", "evictable", "prefix_hits"):
                assert st[k] == so[k], k
        assert ref.prefix_hits > 0


def test_swap_blocks_between_two_pools_matches_the_oracle():
    """Random appends, forks, frees and whole-table swaps between a device pool
    and a host pool, plus requests that must fail (repeated, unheld ids):
    pairs, counts, free lists and errors agree after every operation."""
    for seed in range(3):
        rnd = random.Random(300 + seed)
        ng, nc = rnd.choice([(24, 16), (64, 64)])
        og = np.random.default_rng(seed).permutation(ng).astype(np.int32)
        oc = np.random.default_rng(seed + 50).permutation(nc).astype(np.int32)
        rg, rc = opool.BlockPool(ng, og), opool.BlockPool(nc, oc)
        lg, lc = pa.Pool(ng, og), pa.Pool(nc, oc)
        seqs = []  # [tier, table]
        for _ in range(1200):
            op = rnd.random()
            if op < 0.3:
                t = []
                n = rnd.randint(1, 60)
                row = np.zeros(8, np.int32)
                out_ref, e_ref = _err(lambda: rg.append(t, 0, n, max_blocks=8))
                out_lib, e_lib = _err(lambda: lg.append_slots(row, 0, 0, n))
                assert e_ref == e_lib
                if e_ref is None:
                    assert row[:out_lib[1]].tolist() == t
                    seqs.append(["g", t])
            elif op < 0.4 and seqs:
                tier, t = rnd.choice(seqs)
                ref, lib = (rg, lg) if tier == "g" else (rc, lc)
                seqs.append([tier, ref.fork(t)])
                lib.fork(t)
            elif op < 0.8 and seqs:
                sq = rnd.choice(seqs)
                tier, t = sq
                (rs, rd, ls, ld) = (rg, rc, lg, lc) if tier == "g" else (rc, rg, lc, lg)
                blocks = list(t)
                bad = rnd.random() < 0.15
                if bad:  # a block listed more often than it is held, or not held at all
                    once = [b for b in t if rs.refcount[b] == 1]
                    free = [b for b in range(rs.num_blocks) if rs.refcount[b] == 0]
                    blocks.append(rnd.choice(once + free + [rs.num_blocks + 1]))
                out_ref, e_ref = _err(lambda: opool.swap_blocks(rs, rd, blocks))
                out_lib, e_lib = _err(lambda: pa.swap_blocks(ls, ld, blocks))
                assert e_ref == e_lib, (e_ref, e_lib)
                assert (e_ref == "BadBlock") == bad
                if e_ref is None:
                    assert out_lib.tolist() == [list(p) for p in out_ref]
                    sq[0] = "c" if tier == "g" else "g"
                    sq[1] = [d for _, d in out_ref]
            elif seqs:
                tier, t = seqs.pop(rnd.randrange(len(seqs)))
                (lg if tier == "g" else lc).free_table(t)
                (rg if tier == "g" else rc).free_table(t)  # empties t: the library goes first
            assert [lg.refcount(b) for b in range(ng)] == rg.refcount
            assert [lc.refcount(b) for b in range(nc)] == rc.refcount
            assert lg.num_free() == rg.num_free() and lc.num_free() == rc.num_free()
