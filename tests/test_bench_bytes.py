"""The bench's byte accounting: the cached positions one decode call reads,
counting a physical block shared by several block tables once (hand-counted
cases; the closed form without sharing)."""
import numpy as np

import bench


def test_no_sharing_counts_every_position():
    lens = [1, 16, 17, 40]
    rows = np.array([[0, 0, 0], [1, 0, 0], [2, 3, 0], [4, 5, 6]])
    assert bench.unique_kv_tokens(lens, rows) == sum(lens)


def test_shared_full_block_counts_once():
    # A: block 5 (16 positions) then block 6 (4); B: block 5 shared, then 7 (2)
    lens = [20, 18]
    rows = np.array([[5, 6], [5, 7]])
    assert bench.unique_kv_tokens(lens, rows) == 16 + 4 + 2


def test_shared_partial_block_counts_its_fullest_use():
    # both tables point at block 3; one attends 10 of its positions, one 14
    lens = [10, 14]
    rows = np.array([[3], [3]])
    assert bench.unique_kv_tokens(lens, rows) == 14


def test_empty_sequences_read_nothing():
    assert bench.unique_kv_tokens([0, 0], np.zeros((2, 1), dtype=int)) == 0
