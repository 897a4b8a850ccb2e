"""Pins of oracle.cache_ops on hand-written tiny caches."""
import numpy as np

from oracle import cache_ops


def _cache(nb=3, h=2, d=2):
    return np.zeros((nb, h, 16, d), np.uint16), np.zeros((nb, h, 16, d), np.uint16)


def test_reshape_and_cache_places_rows_by_slot():
    kc, vc = _cache()
    key = np.array([[[1, 2], [3, 4]], [[5, 6], [7, 8]], [[9, 9], [9, 9]]], np.uint16)
    val = key + 100
    cache_ops.reshape_and_cache(key, val, kc, vc, [17, 47, -1])
    # slot 17 = block 1 row 1; slot 47 = block 2 row 15; slot -1 is skipped
    assert kc[1, 0, 1].tolist() == [1, 2] and kc[1, 1, 1].tolist() == [3, 4]
    assert kc[2, 0, 15].tolist() == [5, 6] and kc[2, 1, 15].tolist() == [7, 8]
    assert vc[1, 1, 1].tolist() == [103, 104] and vc[2, 0, 15].tolist() == [105, 106]
    assert int((kc != 0).sum()) == 8 and int((vc != 0).sum()) == 8
    assert not np.any(kc == 9)


def test_copy_blocks_then_write_keeps_the_pre_write_contents():
    kc, vc = _cache(nb=4)
    kc[1] = 7
    vc[1] = 8
    # a shared partial block 1: the copy is taken first, then the in-place writer writes
    cache_ops.copy_blocks(kc, vc, [(1, 3)])
    cache_ops.reshape_and_cache(np.full((1, 2, 2), 5, np.uint16), np.full((1, 2, 2), 6, np.uint16),
                                kc, vc, [1 * 16 + 4])
    assert np.all(kc[3] == 7) and np.all(vc[3] == 8)
    assert np.all(kc[1, :, 4] == 5) and np.all(kc[1, :, 5] == 7)
    assert np.all(kc[0] == 0) and np.all(kc[2] == 0)


def test_copy_blocks_pairs_in_order():
    kc, vc = _cache(nb=4)
    for b in range(4):
        kc[b] = b
        vc[b] = 10 + b
    cache_ops.copy_blocks(kc, vc, np.array([[0, 2], [3, 1]]))
    assert [int(kc[b, 0, 0, 0]) for b in range(4)] == [0, 3, 0, 3]
    assert [int(vc[b, 0, 0, 0]) for b in range(4)] == [10, 13, 10, 13]
