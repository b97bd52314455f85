"""Pins for the Python block-manager model against the pages' printed values
and the invariants they state."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_pins.json")))


def test_widget_tables_are_reproduced():
    w = GOLDEN["widget_tables"]
    bm = oracle.BlockManagerModel(w["num_blocks"], w["block_size"])
    for r, L in enumerate(w["lengths"]):
        bm.append(r, L)
    assert [bm.table(r) for r in range(len(w["lengths"]))] == w["tables"]
    bm.check()


def test_widget_statistics_arithmetic():
    """Fourteen running sequences holding 213 live tokens in 58 blocks of 4.
    The six tables the page shows are used as printed; the other eight
    lengths are a construction of this test (the page does not show them)
    chosen to match the printed totals."""
    w = GOLDEN["widget_stats"]
    lengths = GOLDEN["widget_tables"]["lengths"] + [13, 13, 13, 16, 16, 16, 20, 20]
    bm = oracle.BlockManagerModel(w["num_blocks"], w["block_size"])
    for r, L in enumerate(lengths):
        bm.append(r, L)
    st = bm.stats()
    assert st["num_seqs"] == w["running"]
    assert st["used_blocks"] == w["used_blocks"]
    assert st["logical_tokens"] == w["live_tokens"]
    in_used = 1 - st["logical_tokens"] / (st["used_blocks"] * w["block_size"])
    whole = 1 - st["logical_tokens"] / (st["num_blocks"] * w["block_size"])
    assert round(100 * in_used) == w["waste_in_used_blocks_pct"]
    assert round(100 * whole) == w["wasted_pct"]


def test_reply_of_200_tokens():
    p = GOLDEN["reply_200"]
    bm = oracle.BlockManagerModel(300, p["block_size"])
    bm.append(0, p["length"])
    assert len(bm.table(0)) == p["blocks"]
    slots = len(bm.table(0)) * p["block_size"]
    assert slots == p["slots"] and slots - p["length"] == p["wasted_slots"]
    assert 100 * p["wasted_slots"] / p["slots"] < p["paged_waste_below_pct"]
    bm.append(1, p["contiguous_reservation"])
    assert len(bm.table(1)) == p["reserved_blocks_at_4096"]
    wasted = p["contiguous_reservation"] - p["length"]
    assert wasted == p["contiguous_wasted"]
    assert 100 * wasted / p["contiguous_reservation"] > p["contiguous_waste_above_pct"]


def test_reservation_waste_and_capacity_arithmetic():
    r = GOLDEN["reservation_40_of_2048"]
    assert round(100 * (1 - r["used"] / r["reserved"])) == r["waste_pct"]
    c = GOLDEN["capacity"]
    per_token = c["per_token_kib"] * 1024
    assert c["reservation_tokens"] * per_token == c["reservation_gib"] * 2**30
    slots = c["cache_gib"] * 2**30 // per_token
    assert slots // c["reservation_tokens"] == c["contiguous_requests"]
    per_seq = math.ceil(c["reply_tokens"] / c["block_size"]) * c["block_size"]
    paged = slots // per_seq
    assert abs(paged - c["paged_sequences_approx"]) / c["paged_sequences_approx"] < 0.05


@pytest.mark.parametrize("lengths,blocks,tails", [([1, 17, 33, 100], [1, 2, 3, 7], [15, 15, 15, 12])])
def test_block_counts_and_tail_waste_small_case(lengths, blocks, tails):
    bm = oracle.BlockManagerModel(64, 16, np.random.default_rng(1).permutation(64))
    for s, L in enumerate(lengths):
        bm.append(s, L)
    assert [len(bm.table(s)) for s in range(4)] == blocks
    assert [16 * len(bm.table(s)) - L for s, L in enumerate(lengths)] == tails


def test_tail_waste_bound_and_mean():
    t = GOLDEN["tail_waste"]
    b = t["block_size"]
    rng = np.random.default_rng(11)
    lengths = rng.integers(1, 5000, size=20000)
    bm = oracle.BlockManagerModel(int(lengths.sum()) // b + len(lengths) + 1, b)
    waste = []
    for s, L in enumerate(lengths[:4000]):
        bm.append(s, int(L))
        waste.append(b * len(bm.table(s)) - int(L))
    waste = np.array(waste)
    assert waste.min() >= 0 and waste.max() <= t["max"]
    assert waste.mean() < t["expected_below"]
    assert abs(waste.mean() - t["expected_approx"]) < 1.0


def test_fork_and_prune_refcounts():
    p = GOLDEN["beam_prune"]
    bm = oracle.BlockManagerModel(100, 16)
    bm.append(0, 40)
    prefix = bm.table(0)
    for c in range(1, p["branches"]):
        bm.fork(0, c)
    assert all(bm.refcount[b] == p["branches"] for b in prefix)
    bm.free_seq(3)
    assert all(bm.refcount[b] == p["after_prune"] for b in prefix)
    assert all(b not in bm.free for b in prefix)
    bm.check()


def test_retire_returns_only_blocks_reaching_zero():
    bm = oracle.BlockManagerModel(50, 4)
    bm.append(0, 10)       # blocks 0,1,2 (last partial)
    bm.fork(0, 1)
    slots, cow = bm.append(1, 1)   # writes into shared block 2 -> copy
    assert cow == [(2, 3)] and slots == [3 * 4 + 2]
    bm.append(1, 5)
    before = set(bm.free)
    bm.free_seq(1)
    returned = set(bm.free) - before
    assert returned == {3, 4}
    assert all(bm.refcount[b] == 1 for b in bm.table(0))
    bm.check()
    bm.free_seq(12345)     # unknown sequence: no-op
    bm.check()


def test_shared_prompt_footprint():
    sp = GOLDEN["shared_prompt"]
    b = 16
    bm = oracle.BlockManagerModel(1000, b)
    bm.append(0, sp["prompt_tokens"])
    for j in range(1, sp["samples"]):
        bm.fork(0, j)
    used = bm.stats()["used_blocks"]
    assert used == sp["prompt_tokens"] // b == 125
    assert used * b == sp["tokens_shared_approx"]
    assert sp["samples"] * sp["prompt_tokens"] == sp["tokens_private"]
    # 2000 is a multiple of 16: the next token of every sample opens a fresh
    # block and nothing is copied.
    _, cows = bm.append_step(range(sp["samples"]))
    assert cows == [] and bm.stats()["used_blocks"] == 125 + sp["samples"]
    bm.check()


def test_exercise_four_samples_of_a_1000_token_prompt():
    e = GOLDEN["exercise_1000x4"]
    b = e["block_size"]
    bm = oracle.BlockManagerModel(1000, b)
    bm.append(0, e["prompt_tokens"])
    for j in range(1, e["samples"]):
        bm.fork(0, j)
    _, cows = bm.append_step(range(e["samples"]))
    assert len(cows) == e["samples"] - 1     # last holder writes in place
    slots_held = bm.stats()["used_blocks"] * b
    assert slots_held == (63 + 3) * b
    assert abs(slots_held - e["approx_shared"]) < 0.1 * e["approx_shared"]
    assert slots_held < e["private"] / 3
    bm.check()


def test_out_of_blocks_changes_nothing():
    bm = oracle.BlockManagerModel(4, 4)
    bm.append(0, 9)
    snapshot = (list(bm.free), list(bm.refcount), bm.table(0), bm.length(0))
    with pytest.raises(oracle.OutOfBlocks):
        bm.append(0, 8)
    with pytest.raises(oracle.OutOfBlocks):
        bm.append(1, 5)
    assert (list(bm.free), list(bm.refcount), bm.table(0), bm.length(0)) == snapshot
    assert bm.stats()["alloc_failures"] == 2
    bm.append(1, 4)
    bm.check()


def test_random_operation_sequences_keep_counts_exact():
    """After every operation each block's count equals the number of tables
    naming it (S06 'Reference counts must be exact')."""
    rng = np.random.default_rng(12)
    for trial in range(20):
        b = int(rng.choice([1, 2, 4, 8, 16]))
        bm = oracle.BlockManagerModel(int(rng.integers(8, 80)), b, None)
        live = []
        nxt = 0
        for _ in range(200):
            op = rng.integers(0, 4)
            try:
                if op == 0 or not live:
                    bm.append(nxt, int(rng.integers(0, 3 * b)))
                    live.append(nxt)
                    nxt += 1
                elif op == 1:
                    bm.append(int(rng.choice(live)), int(rng.integers(0, 2 * b)))
                elif op == 2:
                    bm.fork(int(rng.choice(live)), nxt)
                    live.append(nxt)
                    nxt += 1
                else:
                    s = int(rng.choice(live))
                    bm.free_seq(s)
                    live.remove(s)
            except oracle.OutOfBlocks:
                pass
            bm.check()


def test_append_step_is_all_or_nothing_and_handles_shared_tails():
    bm = oracle.BlockManagerModel(6, 4)
    bm.append(0, 3)
    bm.fork(0, 1)
    bm.fork(0, 2)
    # Block 0 is shared three ways: the first two writers copy, the last one
    # writes in place.
    slots, cows = bm.append_step([0, 1, 2])
    assert len(cows) == 2 and [c[0] for c in cows] == [0, 0]
    assert bm.refcount[0] == 1 and bm.table(2) == [0]
    assert slots[2] == 3
    bm.check()
    # Three blocks used, three free; the next step opens a block per sequence
    # and fits exactly, the one after writes inside those blocks.
    bm.append_step([0, 1, 2])
    assert len(bm.free) == 0
    snapshot = (list(bm.free), list(bm.refcount), [bm.table(s) for s in range(3)])
    with pytest.raises(oracle.OutOfBlocks):
        bm.append_step([0, 1, 2, 7])       # sequence 7 would need a block
    assert (list(bm.free), list(bm.refcount), [bm.table(s) for s in range(3)]) == snapshot
    bm.append_step([0, 1, 2])
    bm.check()


def test_append_step_exact_capacity():
    bm = oracle.BlockManagerModel(6, 4)
    bm.append(0, 4)
    bm.append(1, 4)
    bm.append(2, 4)
    slots, cows = bm.append_step([0, 1, 2])
    assert cows == [] and len(bm.free) == 0
    with pytest.raises(oracle.OutOfBlocks):
        bm.append(3, 1)
    bm.check()
