"""Pins of oracle.accounting against the numbers the pages print (tests/golden)."""
import json
import os

import pytest

from oracle import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_kv_bytes_per_token_llama3_70b():
    g = _golden("kv_size.json")["per_token"]
    b = acc.kv_bytes(g["num_layers"], 1, g["num_kv_heads"], g["head_dim"], g["precision_bytes"])
    assert b == g["printed_bytes"]
    assert b == g["printed_kib"] * 1024


@pytest.mark.parametrize("case", _golden("kv_size.json")["totals"], ids=lambda c: c["model"])
def test_kv_bytes_totals(case):
    b = acc.kv_bytes(case["num_layers"], case["seq_length"], case["num_kv_heads"],
                     case["head_dim"], case["precision_bytes"])
    assert b == case["exact_bytes"]
    # the printed figure is the byte count over 2**20, then over 1000
    printed = float(case["printed"].split()[0])
    assert printed == pytest.approx(b / 2**20 / 1000, rel=1e-9)


def test_llama3_8b_table_is_the_equation_at_four_bytes():
    g = _golden("kv_size.json")["llama3_8b_table"]
    for tokens, gb in g["printed_gb"]:
        fp32 = acc.kv_bytes(g["num_layers"], tokens, g["num_kv_heads"], g["head_dim"], 4)
        fp16 = acc.kv_bytes(g["num_layers"], tokens, g["num_kv_heads"], g["head_dim"], 2)
        assert round(fp32 / 1e9, 2) == gb
        assert round(fp16 / 1e9, 2) != gb or tokens == 0


def test_per_request_and_256_users():
    g = _golden("kv_size.json")["per_request_4096"]
    b = acc.kv_bytes(g["num_layers"], g["seq_length"], g["num_kv_heads"], g["head_dim"],
                     g["precision_bytes"])
    assert b == 1_342_177_280
    assert round(b / 1e9, 1) == g["printed_gb_approx"]
    # the page's total is the rounded figure times the users; within 3 %
    assert abs(b * g["users"] / 1e9 - g["printed_total_gb"]) / (b * g["users"] / 1e9) < 0.03


def test_blocks_needed_brute_force():
    for n in range(0, 200):
        # count blocks by filling 16-slot shelves one token at a time
        blocks, free_slots = 0, 0
        for _ in range(n):
            if free_slots == 0:
                blocks += 1
                free_slots = 16
            free_slots -= 1
        assert acc.blocks_needed(n) == blocks
        assert acc.paged_waste(n) == free_slots
        assert 0 <= acc.paged_waste(n) < 16


def test_shelf_and_reservation_examples():
    g = _golden("blocks.json")
    assert acc.blocks_needed(g["shelf_example"]["tokens"]) == g["shelf_example"]["blocks"]
    r = g["reservation_example"]
    assert acc.contiguous_waste(r["used"], r["reserved"]) == r["idle"]
    f = g["internal_fragmentation"]
    idle = acc.contiguous_waste(f["used"], f["reserved"])
    assert round(100 * idle / f["reserved"]) == f["printed_waste_percent"]
    # paged storage of the same request idles only the last block's tail
    assert acc.paged_waste(300) == 4


def test_waste_fraction_and_pool_sizing():
    assert acc.waste_fraction([16, 32]) == 0.0
    assert acc.waste_fraction([1]) == pytest.approx(15 / 16)
    # one block of all 80 layers of Llama 3 70B holds 16 x 327,680 bytes
    assert acc.blocks_for_bytes(16 * 327_680, 80, 8, 128, 2) == 1
    assert acc.blocks_for_bytes(16 * 327_680 - 1, 80, 8, 128, 2) == 0
    # 2048 blocks per 32K sequence: the long-context workload's KV check
    assert 2048 * 16 * 327_680 == acc.kv_bytes(80, 32768, 8, 128, 2)
