"""Pins for the oracle's swap path: the block-manager model's swap-out and
swap-in bookkeeping and the byte copy between a device pool and a host pool.

The pages give preemption by copying a sequence's cache to host memory and
back as the alternative to recomputing it, and ask for it to be built once
the allocator can be driven dry (mercemay.com "Paged KV Cache Allocation and
the Block Table", "Three ways contiguous reservation loses memory";
llminference.xinbetween.com S06, third exercise).  What is fixed without any
further reading: after a round trip every sequence reads exactly the keys and
values it read before, counts stay exact, and a call that does not fit
changes nothing.  The free-list order of the hand-worked example follows the
model's stated discipline (ascending at first, last retired reused first).
"""
import numpy as np
import pytest

import oracle


def _snapshot(bm):
    return (list(bm.free), list(bm.refcount), list(bm.host_free), list(bm.host_refcount),
            {s: bm.table(s) for s in bm.lengths}, dict(bm.lengths))


def test_hand_worked_swap_out_and_in():
    bm = oracle.BlockManagerModel(8, 4)
    bm.set_host_blocks(6)
    bm.append(0, 10)                      # blocks 0, 1, 2
    bm.append(1, 5)                       # blocks 3, 4
    pairs = bm.swap_out([0])
    assert pairs == [(0, 0), (1, 1), (2, 2)]
    assert bm.is_swapped(0) and not bm.is_swapped(1)
    assert bm.table(0) == [0, 1, 2] and bm.length(0) == 10
    # Retired in table order: block 2 is on top and is handed out next.
    assert bm.free == [7, 6, 5, 0, 1, 2]
    bm.append(1, 4)                       # length 9: position 8 opens a block
    assert bm.table(1) == [3, 4, 2]
    pairs = bm.swap_in([0])
    assert pairs == [(0, 1), (1, 0), (2, 5)]
    assert bm.table(0) == [1, 0, 5] and not bm.is_swapped(0)
    assert bm.host_free == [5, 4, 3, 0, 1, 2]
    st = bm.stats()
    assert (st["swap_out_blocks"], st["swap_in_blocks"], st["swapped_seqs"]) == (3, 3, 0)
    assert (st["host_blocks"], st["free_host_blocks"]) == (6, 6)
    bm.check()


def test_swapped_samples_keep_sharing_on_the_host():
    # Four samples of one 1,000-token prompt (the S06 first exercise) swapped
    # out together hold the prompt's blocks once on the host, not four times.
    b = 16
    bm = oracle.BlockManagerModel(1000, b)
    bm.set_host_blocks(1000)
    bm.append(0, 1000)
    for j in range(1, 4):
        bm.fork(0, j)
    bm.append_step(range(4))
    used = bm.stats()["used_blocks"]
    assert used == 63 + 3
    pairs = bm.swap_out(range(4))
    assert len(pairs) == used
    st = bm.stats()
    assert st["used_blocks"] == 0 and st["free_host_blocks"] == 1000 - used
    assert max(bm.host_refcount) == 4
    bm.swap_in(range(4))
    assert bm.stats()["used_blocks"] == used
    assert bm.table(0)[:62] == bm.table(3)[:62]
    bm.check()


def test_block_still_named_by_a_resident_sequence_is_copied_and_kept():
    bm = oracle.BlockManagerModel(6, 4)
    bm.set_host_blocks(4)
    bm.append(0, 8)
    bm.fork(0, 1)
    pairs = bm.swap_out([1])
    assert pairs == [(0, 0), (1, 1)]
    assert bm.refcount[:2] == [1, 1] and bm.table(0) == [0, 1]
    assert bm.stats()["used_blocks"] == 2
    bm.check()
    bm.free_seq(1)                        # releases the host copies only
    assert bm.host_refcount == [0] * 4 and bm.stats()["num_seqs"] == 1
    bm.check()


def test_swap_is_all_or_nothing():
    bm = oracle.BlockManagerModel(6, 4)
    bm.set_host_blocks(2)
    bm.append(0, 9)                       # three blocks: too many for the host
    snap = _snapshot(bm)
    with pytest.raises(oracle.OutOfBlocks):
        bm.swap_out([0])
    assert _snapshot(bm) == snap
    bm.set_host_blocks(3)
    bm.swap_out([0])
    bm.append(1, 20)                      # five of six device blocks
    snap = _snapshot(bm)
    with pytest.raises(oracle.OutOfBlocks):
        bm.swap_in([0])
    assert _snapshot(bm) == snap
    bm.free_seq(1)
    bm.swap_in([0])
    bm.check()


def test_swapped_sequence_cannot_grow_or_fork():
    bm = oracle.BlockManagerModel(6, 4)
    bm.set_host_blocks(6)
    bm.append(0, 5)
    bm.swap_out([0])
    with pytest.raises(ValueError):
        bm.append(0, 1)
    with pytest.raises(ValueError):
        bm.append_step([0])
    with pytest.raises(ValueError):
        bm.fork(0, 1)
    with pytest.raises(ValueError):
        bm.set_host_blocks(8)             # host pool is in use
    with pytest.raises(KeyError):
        bm.swap_out([0])                  # not resident
    with pytest.raises(ValueError):
        bm.swap_in([0, 0])


def _fill(bm, pool_k, pool_v, seqs, rng):
    """Write random rows for every position of the listed resident sequences."""
    for s in seqs:
        n = bm.length(s)
        slots = np.array([oracle.slot_address(bm.table(s), t, bm.block_size) for t in range(n)])
        shape = (n,) + pool_k.shape[2:]
        oracle.reshape_and_cache(pool_k, pool_v, rng.standard_normal(shape), rng.standard_normal(shape), slots)


def _read(bm, k, v, s):
    return (oracle.gather_logical(k, np.array(bm.table(s)), bm.length(s), bm.block_size),
            oracle.gather_logical(v, np.array(bm.table(s)), bm.length(s), bm.block_size))


def test_round_trip_restores_every_key_and_value_bitwise():
    """Preempt, let other sequences overwrite the freed blocks, restore:
    the restored sequences read the same bytes and give the same attention."""
    rng = np.random.default_rng(5)
    b, hkv, d, hq = 4, 2, 8, 4
    bm = oracle.BlockManagerModel(24, b, rng.permutation(24))
    bm.set_host_blocks(16)
    k = np.zeros((24, b, hkv, d))
    v = np.zeros((24, b, hkv, d))
    hk = np.full((16, b, hkv, d), np.nan)
    hv = np.full((16, b, hkv, d), np.nan)
    bm.append(0, 13)
    bm.fork(0, 1)
    _, cows = bm.append(1, 6)             # first write copies the shared partial block
    assert len(cows) == 1
    _fill(bm, k, v, [0], rng)
    for blk_src, blk_dst in zip(bm.table(0), bm.table(1)):
        if blk_src != blk_dst:
            k[blk_dst], v[blk_dst] = k[blk_src], v[blk_src]
    # Sample 1's own positions get fresh rows.
    n1 = bm.length(1)
    slots = np.array([oracle.slot_address(bm.table(1), t, b) for t in range(13, n1)])
    oracle.reshape_and_cache(k, v, rng.standard_normal((len(slots), hkv, d)),
                             rng.standard_normal((len(slots), hkv, d)), slots)
    bm.append(2, 7)
    _fill(bm, k, v, [2], rng)
    before = {s: _read(bm, k, v, s) for s in (0, 1, 2)}
    q = rng.standard_normal((3, hq, d))
    att_before = [oracle.attend(q[s], *before[s], 0.3) for s in (0, 1, 2)]

    out_pairs = bm.swap_out([0, 1])
    oracle.swap_blocks(k, v, hk, hv, np.array(out_pairs))
    # Other work reuses the freed device blocks and overwrites them.
    bm.append(3, 4 * len(bm.free))
    k[bm.table(3)] = -7.0
    v[bm.table(3)] = 9.0
    bm.free_seq(3)
    in_pairs = bm.swap_in([1, 0])
    oracle.swap_blocks(hk, hv, k, v, np.array(in_pairs))
    bm.check()
    for s in (0, 1, 2):
        ks, vs = _read(bm, k, v, s)
        assert np.array_equal(ks, before[s][0]) and np.array_equal(vs, before[s][1])
        assert np.array_equal(oracle.attend(q[s], ks, vs, 0.3), att_before[s])
    # Swapped together, the two samples share their common blocks again.
    assert bm.table(0)[:3] == bm.table(1)[:3]


def test_swap_blocks_moves_whole_blocks_of_both_pools_only():
    rng = np.random.default_rng(2)
    src_k = rng.standard_normal((5, 4, 2, 8)).astype(np.float32)
    src_v = rng.standard_normal((5, 4, 2, 8)).astype(np.float32)
    dst_k = np.zeros((3, 4, 2, 8), np.float32)
    dst_v = np.zeros((3, 4, 2, 8), np.float32)
    oracle.swap_blocks(src_k, src_v, dst_k, dst_v, np.array([[4, 0], [1, 2]]))
    assert np.array_equal(dst_k[0], src_k[4]) and np.array_equal(dst_v[0], src_v[4])
    assert np.array_equal(dst_k[2], src_k[1]) and np.array_equal(dst_v[2], src_v[1])
    assert not dst_k[1].any() and not dst_v[1].any()
    with pytest.raises(ValueError):
        oracle.swap_blocks(src_k, src_v, dst_k, dst_v, np.array([[0, 1], [2, 1]]))
    with pytest.raises(ValueError):
        oracle.swap_blocks(src_k, src_v, dst_k, dst_v, np.array([[0, 3]]))
    with pytest.raises(ValueError):
        oracle.swap_blocks(src_k, src_v, dst_k[:, :2], dst_v[:, :2], np.array([[0, 0]]))


def test_random_operations_with_swaps_keep_counts_exact():
    rng = np.random.default_rng(31)
    for trial in range(15):
        b = int(rng.choice([1, 2, 4, 8, 16]))
        bm = oracle.BlockManagerModel(int(rng.integers(8, 60)), b, None)
        bm.set_host_blocks(int(rng.integers(0, 60)))
        resident, swapped, nxt = [], [], 0
        for _ in range(200):
            op = int(rng.integers(0, 6))
            try:
                if op == 0 or not (resident or swapped):
                    bm.append(nxt, int(rng.integers(0, 3 * b)))
                    resident.append(nxt)
                    nxt += 1
                elif op == 1 and resident:
                    bm.append(int(rng.choice(resident)), int(rng.integers(0, 2 * b)))
                elif op == 2 and resident:
                    bm.fork(int(rng.choice(resident)), nxt)
                    resident.append(nxt)
                    nxt += 1
                elif op == 3 and resident:
                    k = int(rng.integers(1, len(resident) + 1))
                    pick = [int(x) for x in rng.choice(resident, size=k, replace=False)]
                    bm.swap_out(pick)
                    for s in pick:
                        resident.remove(s)
                        swapped.append(s)
                elif op == 4 and swapped:
                    k = int(rng.integers(1, len(swapped) + 1))
                    pick = [int(x) for x in rng.choice(swapped, size=k, replace=False)]
                    bm.swap_in(pick)
                    for s in pick:
                        swapped.remove(s)
                        resident.append(s)
                elif op == 5:
                    pool = resident + swapped
                    s = int(rng.choice(pool))
                    bm.free_seq(s)
                    (resident if s in resident else swapped).remove(s)
            except oracle.OutOfBlocks:
                pass
            bm.check()
