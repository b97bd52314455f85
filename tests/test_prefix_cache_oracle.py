"""Pins for the oracle's prefix cache across requests (the block-manager model).

The pages: a chat server sends the same system prompt over and over; hashing
block contents lets any two requests with a common prefix share the same
physical blocks, and prefill cost often drops by an order of magnitude
(llminference.xinbetween.com S06, "What's next"; "Unshareable duplicates": two
requests with the same 2,000-token system prompt otherwise hold two copies).
What is fixed without further reading: a reused block holds exactly the keys
and values a private prefill would have written, so every request reads the
same rows and gets the same attention; sharing follows the prefix, not a
block's own tokens; counts stay exact.  Free-list and eviction orders in the
hand-worked examples follow the model's stated discipline.
"""
import numpy as np
import pytest

import oracle
import synth


def _snapshot(bm):
    return (list(bm.free), list(bm.refcount), dict(bm.evictable), dict(bm.index),
            {s: bm.table(s) for s in bm.lengths}, dict(bm.lengths))


def test_two_requests_with_one_2000_token_system_prompt():
    b = 16
    rng = np.random.default_rng(0)
    system = rng.integers(0, 32000, size=2000)
    bm = oracle.BlockManagerModel(400, b)
    bm.enable_prefix_cache()
    a = np.concatenate([system, rng.integers(0, 32000, size=100)])
    c = np.concatenate([system, rng.integers(0, 32000, size=120)])
    slots_a, cached_a = bm.append_prompt(0, a)
    slots_c, cached_c = bm.append_prompt(1, c)
    assert cached_a == 0 and cached_c == 2000
    assert slots_c[:2000] == [-1] * 2000 and min(slots_c[2000:]) >= 0
    # 125 shared system blocks, 7 + 8 private ones, instead of 132 + 133.
    assert bm.stats()["used_blocks"] == 125 + 7 + 8
    assert bm.table(1)[:125] == bm.table(0)[:125] and bm.table(1)[125] != bm.table(0)[125]
    # Prefill for the second request computes 120 of 2,120 tokens.
    assert len(c) / (len(c) - cached_c) > 10
    st = bm.stats()
    assert (st["prefix_query_tokens"], st["prefix_hit_tokens"]) == (2100 + 2120, 2000)
    bm.check()


def test_identical_prompt_leaves_its_last_token_to_compute():
    b = 16
    prompt = np.arange(2000) % 97
    bm = oracle.BlockManagerModel(300, b)
    bm.enable_prefix_cache()
    bm.append_prompt(0, prompt)
    assert bm.stats()["cached_blocks"] == 125
    slots, cached = bm.append_prompt(1, prompt)
    assert cached == 124 * b                      # (2000 - 1) // 16 blocks reused
    assert all(s >= 0 for s in slots[1984:]) and bm.table(1)[124] != bm.table(0)[124]
    assert bm.stats()["cached_blocks"] == 125     # the duplicate last block is not indexed twice
    bm.check()


@pytest.mark.parametrize("p", [0, 3, 4, 5, 11, 12, 23])
def test_reuse_stops_at_the_first_block_that_differs(p):
    b = 4
    base = list(range(100, 125))                  # 25 tokens
    other = list(base)
    other[p] += 1000
    bm = oracle.BlockManagerModel(40, b)
    bm.enable_prefix_cache()
    bm.append_prompt(0, base)
    _, cached = bm.append_prompt(1, other)
    assert cached == (p // b) * b


def test_a_block_is_shared_by_prefix_not_by_its_own_tokens():
    b = 4
    x, y, z = [1, 2, 3, 4], [5, 6, 7, 8], [9, 9, 9, 9]
    bm = oracle.BlockManagerModel(20, b)
    bm.enable_prefix_cache()
    bm.append_prompt(0, x + y + [0])
    _, cached = bm.append_prompt(1, z + y + [0])     # same second block, other first block
    assert cached == 0 and bm.table(1)[1] != bm.table(0)[1]
    _, cached = bm.append_prompt(2, x + y + [1])
    assert cached == 8
    bm.check()


def test_hand_worked_eviction_and_revival():
    b = 4
    bm = oracle.BlockManagerModel(7, b)
    bm.enable_prefix_cache()
    a = [1, 1, 1, 1, 2, 2, 2, 2, 3]                   # two full blocks and one token
    bm.append_prompt(0, a)
    assert bm.table(0) == [0, 1, 2]
    bm.free_seq(0)
    # Block 2 (partial, never cached) goes back on the free list; the cached
    # blocks become evictable deepest first: 1 before 0.
    assert bm.free == [6, 5, 4, 3, 2] and bm.evictable == {1: 0, 0: 1}
    assert bm.stats()["used_blocks"] == 0
    c = list(range(10, 30))                           # 20 tokens, no overlap: 5 blocks
    bm.append_prompt(1, c)
    assert bm.table(1) == [2, 3, 4, 5, 6]             # the free list is used up first
    bm.append(1, 1)                                   # position 20 opens a block: evicts block 1
    assert bm.table(1)[-1] == 1 and bm.evictable == {0: 1}
    # The same prompt again: block 0 is still cached and is revived; block 1's
    # content is gone, so only four tokens are reused.
    snap = _snapshot(bm)
    with pytest.raises(oracle.OutOfBlocks):
        bm.append_prompt(2, a)                        # needs 2 new blocks, 0 left besides the hit
    assert _snapshot(bm) == snap
    bm.free_seq(1)
    slots, cached = bm.append_prompt(2, a)
    assert cached == 4 and bm.table(2)[0] == 0 and slots[:4] == [-1] * 4
    bm.check()


def test_revived_hits_are_charged_against_capacity():
    b = 4
    bm = oracle.BlockManagerModel(4, b)
    bm.enable_prefix_cache()
    bm.append_prompt(0, [1] * 8 + [2])                # blocks 0, 1 cached; 2 private
    bm.free_seq(0)
    bm.append_prompt(1, [7])                           # takes free block 2; block 3 is left
    # Reusing both cached blocks needs one new block; capacity counts the
    # two evictable blocks, but reviving them leaves only the one free block.
    slots, cached = bm.append_prompt(2, [1] * 8 + [5])
    assert cached == 8
    snap = _snapshot(bm)
    with pytest.raises(oracle.OutOfBlocks):
        bm.append_prompt(3, [1] * 8 + [6, 6, 6, 6, 6])  # needs two new blocks, none left
    assert _snapshot(bm) == snap
    bm.check()


@pytest.mark.parametrize("name", ["h1s", "h1f"])
def test_cached_prefill_reads_the_rows_a_private_prefill_writes(name):
    """Requests with shared system prompts, admitted through the cache (only
    non-reused slots written) or privately (every slot written), with
    retirements in between so that evicted blocks are reused: every live
    request reads bit-identical keys and values either way."""
    case = synth.prefix_cache_case(name)
    cfg = case["cfg"]
    b, hkv, d, dt = cfg["block_size"], cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    nb = case["num_blocks"] // 4                      # small enough to retire requests and evict
    bm = oracle.BlockManagerModel(nb, b)
    bm.enable_prefix_cache()
    k = synth.nan_fill((nb, b, hkv, d), dt)
    v = synth.nan_fill((nb, b, hkv, d), dt)
    live = []
    hits = retired = 0
    for r, prompt in enumerate(case["prompts"]):
        while True:
            try:
                slots, cached = bm.append_prompt(r, prompt)
                break
            except oracle.OutOfBlocks:
                bm.free_seq(live.pop(0))
                retired += 1
        hits += cached
        rk, rv = synth.token_rows(prompt, hkv, d, dt)
        oracle.reshape_and_cache(k, v, rk, rv, np.array(slots, dtype=np.int64))
        live.append(r)
        for s in live:
            p = case["prompts"][s]
            ek, ev = synth.token_rows(p, hkv, d, dt)
            gk = oracle.gather_logical(k, np.array(bm.table(s)), len(p), b)
            gv = oracle.gather_logical(v, np.array(bm.table(s)), len(p), b)
            assert np.array_equal(gk, ek) and np.array_equal(gv, ev), (r, s)
        bm.check()
    assert hits > 0 and retired > 0


def test_prefix_cache_errors():
    bm = oracle.BlockManagerModel(8, 4)
    with pytest.raises(ValueError):
        bm.append_prompt(0, [1, 2])                    # cache off
    bm.append(0, 1)
    with pytest.raises(ValueError):
        bm.enable_prefix_cache()                       # sequences exist
    bm.free_seq(0)
    bm.enable_prefix_cache()
    bm.append_prompt(0, [1, 2, 3])
    with pytest.raises(ValueError):
        bm.append_prompt(0, [1, 2, 3])                 # sequence exists
    assert bm.append_prompt(1, []) == ([], 0)


def test_random_operations_with_prefix_cache_keep_counts_exact():
    rng = np.random.default_rng(44)
    for trial in range(12):
        b = int(rng.choice([1, 2, 4, 8]))
        bm = oracle.BlockManagerModel(int(rng.integers(6, 50)), b)
        bm.enable_prefix_cache()
        bm.set_host_blocks(int(rng.integers(0, 40)))
        systems = [list(rng.integers(0, 3, size=int(rng.integers(0, 5 * b)))) for _ in range(3)]
        resident, swapped, nxt = [], [], 0
        for _ in range(200):
            op = int(rng.integers(0, 7))
            try:
                if op <= 1 or not (resident or swapped):
                    sysp = systems[int(rng.integers(0, 3))]
                    prompt = sysp + list(rng.integers(0, 3, size=int(rng.integers(0, 3 * b))))
                    bm.append_prompt(nxt, prompt)
                    resident.append(nxt)
                    nxt += 1
                elif op == 2 and resident:
                    bm.append(int(rng.choice(resident)), int(rng.integers(0, 2 * b)))
                elif op == 3 and resident:
                    bm.fork(int(rng.choice(resident)), nxt)
                    resident.append(nxt)
                    nxt += 1
                elif op == 4 and resident:
                    s = int(rng.choice(resident))
                    bm.swap_out([s])
                    resident.remove(s)
                    swapped.append(s)
                elif op == 5 and swapped:
                    s = swapped[0]
                    bm.swap_in([s])
                    swapped.remove(s)
                    resident.append(s)
                elif op == 6:
                    pool = resident + swapped
                    s = int(rng.choice(pool))
                    bm.free_seq(s)
                    (resident if s in resident else swapped).remove(s)
            except oracle.OutOfBlocks:
                pass
            bm.check()
