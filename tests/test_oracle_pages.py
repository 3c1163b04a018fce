"""Oracle allocation arithmetic against the numbers the pages print."""
import json
import os

import pytest

from oracle import pa_oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_examples.json")))


@pytest.mark.parametrize("ex", GOLDEN["allocation"], ids=lambda e: f"{e['tokens']}@{e['block_size']}")
def test_blocks_and_slack_printed(ex):
    assert O.blocks_needed(ex["tokens"], ex["block_size"]) == ex["blocks"]
    if "slack" in ex:
        assert O.slack(ex["tokens"], ex["block_size"]) == ex["slack"]


def test_slack_bound_every_length():
    # the last block wastes at most block_size - 1 positions, and the blocks
    # are the fewest that hold the tokens (brute force over lengths)
    for bs in (8, 16, 32, 64, 128):
        for n in range(0, 10001):
            nb = O.blocks_needed(n, bs)
            s = O.slack(n, bs)
            assert 0 <= s <= bs - 1
            assert nb * bs >= n and (nb - 1) * bs < n or n == 0
    g = GOLDEN["max_slack_per_request"]
    assert max(O.slack(n, g["block_size"]) for n in range(1, 2000)) == g["max_slack"]


def test_block_table_example_slots():
    ex = GOLDEN["block_table_example"]
    t, bs = ex["table"], ex["block_size"]
    # positions map to (table[p // bs], p % bs): logical order kept, physical scattered
    assert O.slot_of(t, 0, bs) == 7 * 16
    assert O.slot_of(t, 15, bs) == 7 * 16 + 15
    assert O.slot_of(t, 16, bs) == 2 * 16
    assert O.slot_of(t, 33, bs) == 11 * 16 + 1
    # every position of a 48-token sequence lands in a distinct slot of its block
    slots = [O.slot_of(t, p, bs) for p in range(48)]
    assert len(set(slots)) == 48
    assert [s // bs for s in slots] == [7] * 16 + [2] * 16 + [11] * 16


def test_naive_waste_printed():
    for ex in GOLDEN["naive_waste"]:
        pct = 100.0 * (ex["reserved"] - ex["used"]) / ex["reserved"]
        if "waste_pct" in ex:
            assert pct == ex["waste_pct"]
        else:
            assert int(pct) == ex["waste_pct_rounded"]


def test_capacity_13b_a100():
    c = GOLDEN["capacity_13b_a100"]
    per_tok = O.kv_bytes_per_token(c["num_layers"], c["num_kv_heads"], c["head_dim"], c["elem_bytes"])
    assert per_tok == 819200
    mib = per_tok / 2**20
    assert round(mib, 2) == c["kv_mb_per_token_approx"]
    naive = mib * c["max_context"] / 1024          # GiB reserved per request
    paged = mib * c["answer_tokens"] / 1024
    assert round(naive, 2) == c["naive_gb_per_request_approx"]
    assert round(paged, 3) == c["paged_gb_per_request_approx"]
    assert round(c["kv_budget_gb"] / naive) == c["naive_concurrent_approx"]
    # the page divides by its rounded 0.195 GB
    assert round(c["kv_budget_gb"] / c["paged_gb_per_request_approx"]) == c["paged_concurrent_approx"]
    assert naive / paged == c["ratio_approx"]


def test_chat_workload_arithmetic():
    c = GOLDEN["chat_workload"]
    bs = c["block_size"]
    per_req = O.blocks_needed(800, bs) + O.blocks_needed(200, bs)
    assert per_req == c["blocks_per_request"]
    assert per_req * c["users"] == c["total_blocks"]
    assert bs * c["mb_per_token_as_printed"] == c["mb_per_block"]
    total_mb = c["total_blocks"] * c["mb_per_block"]
    assert abs(total_mb - c["total_mb_approx"]) / c["total_mb_approx"] < 0.01
    shared = O.blocks_needed(500, bs)
    assert shared == c["shared_prompt_blocks"]
    saved_gb = shared * (c["users"] - 1) * c["mb_per_block"] / 1000
    assert round(saved_gb) == c["prefix_savings_gb_approx"]
