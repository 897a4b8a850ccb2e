"""Pins of the oracle pool's prefix cache (oracle.pool: match_prefix, register).

Each test checks the cache against what a prefix cache must do whatever its
keys look like: a matched block holds exactly the query's tokens at its
position (checked against a ledger of what was written where), the number of
matched blocks is the longest common whole-block prefix with a cached
sequence (brute force), cached blocks outlive their sequences until evicted,
and reference counts stay equal to table references.
"""
import random

import numpy as np
import pytest

import workloads
from oracle import step
from oracle.pool import BLOCK_SIZE, BadBlock, BlockPool, InvalidArg, OutOfBlocks, blocks_for


def _conservation(pool, tables):
    counts = [0] * pool.num_blocks
    for t in tables:
        for b in t:
            counts[b] += 1
    assert counts == pool.refcount
    assert sorted(pool.free_stack + pool.lru) == [b for b in range(pool.num_blocks) if counts[b] == 0]
    assert set(pool.lru) <= set(pool.key_of)
    assert not set(pool.free_stack) & set(pool.key_of)


def _lcp(a, b):
    n = 0
    while n < min(len(a), len(b)) and a[n] == b[n]:
        n += 1
    return n


def _new_sequence(pool, tokens, ledger):
    """Prefill through the cache: match, allocate the rest, record what each
    fresh block holds, register.  Returns (table, matched)."""
    table = pool.match_prefix(tokens)
    matched = len(table)
    pos = matched * BLOCK_SIZE
    try:
        slots, cow = pool.append(table, pos, len(tokens) - pos)
    except OutOfBlocks:
        pool.free_table(table)  # give the matched blocks back
        raise
    assert cow is None
    for p, slot in zip(range(pos, len(tokens)), slots):
        ledger[slot] = tokens[p]
    pool.register(table, tokens)
    return table, matched


def test_match_is_the_longest_common_block_prefix_brute_force():
    rnd = random.Random(3)
    pool = BlockPool(4096, free_order=random.Random(4).sample(range(4096), 4096))
    ledger = {}
    seqs = []
    base = [rnd.randrange(50) for _ in range(200)]
    for _ in range(120):
        # share a random-length head of a random earlier sequence (or of base)
        src = rnd.choice([t for t, _ in seqs] + [base]) if seqs else base
        head = src[:rnd.randrange(len(src) + 1)]
        toks = head + [rnd.randrange(3) for _ in range(rnd.randrange(0, 60))]
        if not toks:
            continue
        expect = max([_lcp(toks, t) // BLOCK_SIZE for t, _ in seqs] + [0])
        expect = min(expect, len(toks) // BLOCK_SIZE)
        table, matched = _new_sequence(pool, toks, ledger)
        assert matched == expect
        for p, tok in enumerate(toks):  # every position holds its token
            assert ledger[table[p // BLOCK_SIZE] * BLOCK_SIZE + p % BLOCK_SIZE] == tok
        seqs.append((toks, table))
        _conservation(pool, [t for _, t in seqs])


def test_cached_blocks_outlive_their_sequence():
    pool = BlockPool(16)
    prompt = list(range(40))  # 2 full blocks + 8 tokens
    a, m = _new_sequence(pool, prompt, {})
    assert m == 0 and len(a) == 3 and pool.stats()["cached"] == 2
    pool.free_table(list(a))
    assert pool.refcount[a[0]] == pool.refcount[a[1]] == 0
    assert pool.lru == [a[0], a[1]] and pool.num_free() == 16
    b, m = _new_sequence(pool, prompt, {})
    assert m == 2 and b[:2] == a[:2] and pool.refcount[a[0]] == 1 and not pool.lru
    assert pool.prefix_hits == 2
    _conservation(pool, [b])


def test_uncached_blocks_go_first_then_least_recently_released():
    pool = BlockPool(6, free_order=range(6))
    ledger = {}
    x, _ = _new_sequence(pool, [1] * 32, ledger)  # blocks 0, 1 cached
    y, _ = _new_sequence(pool, [2] * 32, ledger)  # blocks 2, 3 cached
    pool.free_table(list(y))  # released first: 2 then 3
    pool.free_table(list(x))  # then 0, 1
    assert pool.lru == [2, 3, 0, 1] and pool.free_stack == [5, 4]
    got = [pool.alloc() for _ in range(4)]
    assert got == [4, 5, 2, 3]  # uncached (LIFO) first, then oldest releases
    assert pool.stats()["cached"] == 2
    assert pool.match_prefix([2] * 32) == []  # y's blocks were evicted
    z = pool.match_prefix([1] * 32)
    assert z == [0, 1]
    with pytest.raises(OutOfBlocks):
        pool.alloc()


def test_no_false_hit_through_a_reused_block_id():
    pool = BlockPool(3, free_order=[0, 1, 2])
    ledger = {}
    a_toks = [7] * 16 + [8] * 16
    a, _ = _new_sequence(pool, a_toks, ledger)  # blocks 0, 1
    pool.free_table(list(a))
    # evict block 0 only, by taking the one uncached block and then one more
    hold = [pool.alloc(), pool.alloc()]
    assert hold == [2, 0] and pool.match_prefix(a_toks) == []
    pool.free_table(hold)  # 0 and 2 come back uncached
    b_toks = [9] * 16
    b, _ = _new_sequence(pool, b_toks, ledger)  # reuses block id 0 for other tokens
    assert b == [0]
    # block 1 still holds A's second block, but its parent is gone: B's first
    # block followed by A's second chunk must not reach it
    got = pool.match_prefix(b_toks + [8] * 16)
    assert got == [0]
    assert ledger[1 * BLOCK_SIZE] == 8 and pool.refcount[1] == 0


def test_register_is_all_or_nothing():
    pool = BlockPool(8)
    t = []
    pool.append(t, 0, 32)
    before = (dict(pool.cache), list(pool.refcount))
    with pytest.raises(InvalidArg):
        pool.register(t, list(range(48)))  # 3 full chunks, 2 table entries
    freed = pool.alloc()
    pool.free(freed)
    with pytest.raises(BadBlock):
        pool.register([t[0], freed], list(range(32)))
    assert (dict(pool.cache), list(pool.refcount)) == before
    assert pool.register(t, list(range(32))) == 2
    assert pool.register(t, list(range(32))) == 0  # already cached
    with pytest.raises(InvalidArg):
        pool.register(t, list(range(1, 33)))  # a cached block with other tokens


def test_duplicate_content_is_not_cached_twice():
    pool = BlockPool(8)
    toks = [5] * 16 + [6] * 16
    a = []
    pool.append(a, 0, 32)
    b = []
    pool.append(b, 0, 32)
    assert pool.register(a, toks) == 2
    assert pool.register(b, toks) == 0
    assert pool.match_prefix(toks) == a


def test_shared_prompt_block_count_closed_form():
    """64 prompts x 4 samples, prompt = 2048 + t_p tokens (t_p in 1..15),
    through the prefix cache instead of forking: the first sample of a prompt
    allocates all ceil((2048 + t_p)/16) = 129 blocks, the other three match the
    128 whole blocks and allocate their own partial block -- 132 blocks per
    prompt, the same count as fork + copy-on-write."""
    rnd = random.Random(11)
    nprompt, nsample = 64, 4
    pool = BlockPool(64 * 140)
    tables = []
    hits = 0
    for p in range(nprompt):
        prompt = [p * 100_000 + i for i in range(2048 + rnd.randint(1, 15))]
        for _ in range(nsample):
            t, m = _new_sequence(pool, prompt, {})
            tables.append(t)
            hits += m
            assert len(t) == blocks_for(len(prompt))
    used = pool.stats()["used"]
    assert used == nprompt * (129 + (nsample - 1))
    assert hits == nprompt * (nsample - 1) * 128
    assert pool.stats()["cached"] == nprompt * 128
    _conservation(pool, tables)


def test_random_operations_with_prefix_cache_conserve_references():
    rnd = random.Random(21)
    pool = BlockPool(48, free_order=random.Random(22).sample(range(48), 48))
    ledger = {}
    seqs = []  # (table, tokens)
    phrases = [[rnd.randrange(2) for _ in range(BLOCK_SIZE)] for _ in range(3)]
    for _ in range(3000):
        op = rnd.random()
        try:
            if op < 0.35:
                toks = sum((rnd.choice(phrases) for _ in range(rnd.randint(0, 3))), [])
                toks += [rnd.randrange(2) for _ in range(rnd.randint(1, 20))]
                table, _ = _new_sequence(pool, toks, ledger)
                seqs.append((table, toks))
            elif op < 0.6 and seqs:
                i = rnd.randrange(len(seqs))
                table, toks = seqs[i]
                new = [rnd.randrange(2) for _ in range(rnd.randint(1, 20))]
                slots, cow = pool.append(table, len(toks), len(new))
                assert cow is None
                for p, slot in zip(range(len(toks), len(toks) + len(new)), slots):
                    ledger[slot] = new[p - len(toks)]
                toks.extend(new)
                pool.register(table, toks)
            elif seqs:
                table, _ = seqs.pop(rnd.randrange(len(seqs)))
                pool.free_table(table)
        except OutOfBlocks:
            pass
        for table, toks in seqs:
            assert len(table) == blocks_for(len(toks))
            for p, tok in enumerate(toks):
                assert ledger[table[p // BLOCK_SIZE] * BLOCK_SIZE + p % BLOCK_SIZE] == tok
        _conservation(pool, [t for t, _ in seqs])
    assert pool.prefix_hits > 100


@pytest.mark.parametrize("config", [4, "4b"])
def test_shared_prefix_workload_through_the_cache_closed_forms(config):
    """The shared-prefix workloads with their prompts taken from the cache
    instead of forked: every prompt's whole blocks are cached once, every
    later sequence of a prompt hits all of them, nothing is copied, and the
    pool ends with exactly as many blocks in use as fork + copy-on-write."""
    w = workloads.make(config, values=False)
    forked = step.plan(w)
    cached = step.plan(w, prefix_cache=True)
    n_prompts = len(w.prompt_lens)
    per = [int(np.sum(w.prompt_of == p)) for p in range(n_prompts)]
    whole = [int(n) // BLOCK_SIZE for n in w.prompt_lens]
    st = cached.pool.stats()
    assert st["cached"] == sum(whole)
    assert cached.pool.prefix_hits == sum((k - 1) * b for k, b in zip(per, whole))
    assert all(len(ph.pairs) == 0 for ph in cached.phases)
    assert st["used"] == forked.pool.stats()["used"]
    for s in range(w.num_seqs):
        assert len(cached.tables[s]) == blocks_for(int(w.context_lens[s]))


def test_decode_through_the_cache_equals_decode_through_forks():
    """Attention sees only each sequence's K/V, not where the blocks sit:
    the prefix-cached layout decodes bit-identically to the forked one."""
    w = workloads.make_custom([3, 17, 1, 30, 2, 16], hq=4, hkv=2, d=16, dtype="bf16", seed=12,
                              prompt_lens=[37, 32], prompt_of=[0, 0, 0, 1, 1, 1])
    _, _, _, a = step.run(w, np.uint16(0x7FC0))
    _, _, _, b = step.run(w, np.uint16(0x7FC0), prefix_cache=True)
    assert np.array_equal(a, b)
