"""Pins for the float64 attention oracle and the cache-op oracle.

Each check ties the oracle to something other than itself: a closed form, a
library attention routine on the contiguous layout, an invariance the
mathematics fixes, or a value the pages print.  Chosen so that a dropped term,
a wrong head mapping, swapped block/offset arithmetic, a missing scale or a
keys/values mix-up each fails at least one test.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_pins.json")))


def _scatter_contiguous(keys, values, lengths, block_size, num_blocks, rng):
    """Place contiguous per-sequence K/V into a pool through random tables.

    Written independently of the oracle: an explicit loop over blocks that
    copies up to block_size rows at a time into a randomly chosen physical
    block; unused slots stay NaN.
    """
    hkv, d = keys.shape[1:]
    kp = np.full((num_blocks, block_size, hkv, d), np.nan)
    vp = np.full_like(kp, np.nan)
    maxb = max(1, max((int(L) + block_size - 1) // block_size for L in lengths))
    tables = np.full((len(lengths), maxb), -1, dtype=np.int32)
    phys = rng.permutation(num_blocks)
    used = 0
    row = 0
    for s, L in enumerate(lengths):
        start = 0
        j = 0
        while start < L:
            n = min(block_size, L - start)
            blk = phys[used]
            used += 1
            tables[s, j] = blk
            kp[blk, :n] = keys[row + start: row + start + n]
            vp[blk, :n] = values[row + start: row + start + n]
            start += n
            j += 1
        row += L
    tables[tables < 0] = 0
    return kp, vp, tables


def _sdpa(q_s, keys, values, scale):
    """torch float64 scaled_dot_product_attention with grouped KV heads."""
    qt = torch.from_numpy(q_s)[None, :, None, :]            # [1, Hq, 1, D]
    kt = torch.from_numpy(np.ascontiguousarray(keys.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(values.transpose(1, 0, 2)))[None]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, scale=scale, enable_gqa=True)
    return out[0, :, 0, :].numpy()


@pytest.mark.parametrize("hq,hkv,block_size", [(4, 4, 16), (8, 2, 4), (6, 3, 1), (16, 2, 8)])
def test_paged_equals_contiguous_library_attention(hq, hkv, block_size):
    """Paged attention reads the same numbers as contiguous attention
    (S06 'Run it locally': the numerical-equivalence assertion); the library
    routine also fixes the grouped-head convention h -> h // (Hq/Hkv)."""
    rng = np.random.default_rng(100 + hq + block_size)
    d = 32
    lengths = [1, 5, block_size, block_size + 1, 3 * block_size - 1, 37]
    total = sum(lengths)
    keys = rng.standard_normal((total, hkv, d))
    values = rng.standard_normal((total, hkv, d))
    q = rng.standard_normal((len(lengths), hq, d))
    nb = sum(-(-L // block_size) for L in lengths) + 7
    kp, vp, tables = _scatter_contiguous(keys, values, lengths, block_size, nb, rng)
    scale = 0.3
    out = oracle.decode_attention(q, kp, vp, tables, np.array(lengths), scale)
    row = 0
    for s, L in enumerate(lengths):
        ref = _sdpa(q[s], keys[row:row + L], values[row:row + L], float(np.float32(scale)))
        np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)
        row += L


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    keys = rng.standard_normal((1, 2, 8))
    values = rng.standard_normal((1, 2, 8))
    q = rng.standard_normal((4, 8))
    out = oracle.attend(q, keys, values, 0.125)
    for h in range(4):
        assert np.array_equal(out[h], values[0, h // 2])


def test_zero_query_gives_mean_value():
    rng = np.random.default_rng(2)
    keys = rng.standard_normal((23, 1, 16))
    values = rng.standard_normal((23, 1, 16))
    out = oracle.attend(np.zeros((3, 16)), keys, values, 1.0)
    np.testing.assert_allclose(out, np.broadcast_to(values[:, 0].mean(0), (3, 16)), atol=1e-14)


def test_two_tokens_closed_form():
    rng = np.random.default_rng(3)
    keys = rng.standard_normal((2, 1, 8))
    values = rng.standard_normal((2, 1, 8))
    q = rng.standard_normal((1, 8))
    scale = 0.7
    z0, z1 = scale * keys[0, 0] @ q[0], scale * keys[1, 0] @ q[0]
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    expect = sig(z1 - z0) * values[1, 0] + sig(z0 - z1) * values[0, 0]
    np.testing.assert_allclose(oracle.attend(q, keys, values, scale)[0], expect, atol=1e-14)


def test_dominant_logit_selects_its_value_without_overflow():
    """Scores near 1e4 overflow exp() unless the maximum is subtracted."""
    rng = np.random.default_rng(4)
    d = 16
    keys = rng.standard_normal((9, 1, d))
    q = rng.standard_normal((1, d))
    keys[5, 0] = 400.0 * q[0] / np.linalg.norm(q[0])
    values = rng.standard_normal((9, 1, d))
    out = oracle.attend(q, keys, values, 10.0)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[0], values[5, 0], atol=1e-12)


def test_empty_context_gives_zeros():
    q = np.ones((2, 4, 8), dtype=np.float32)
    pool = np.full((3, 4, 2, 8), np.nan, dtype=np.float32)
    out = oracle.decode_attention(q, pool, pool, np.zeros((2, 1), np.int32), np.array([0, 0]), 1.0)
    assert np.array_equal(out, np.zeros_like(out))


def test_token_order_is_irrelevant_but_key_value_pairing_is_not():
    """Attention is a function of the set of (key, value) pairs: permuting
    tokens together leaves it unchanged, permuting values alone changes it."""
    rng = np.random.default_rng(5)
    keys = rng.standard_normal((30, 2, 16))
    values = rng.standard_normal((30, 2, 16))
    q = rng.standard_normal((4, 16))
    perm = rng.permutation(30)
    a = oracle.attend(q, keys, values, 0.25)
    b = oracle.attend(q, keys[perm], values[perm], 0.25)
    c = oracle.attend(q, keys, values[perm], 0.25)
    np.testing.assert_allclose(a, b, atol=1e-13)
    assert np.abs(a - c).max() > 1e-3


def test_output_is_a_convex_combination_of_values():
    rng = np.random.default_rng(6)
    keys = rng.standard_normal((50, 1, 8))
    values = rng.standard_normal((50, 1, 8))
    out = oracle.attend(rng.standard_normal((2, 8)) * 3, keys, values, 1.0)
    assert np.all(out <= values[:, 0].max(0) + 1e-12)
    assert np.all(out >= values[:, 0].min(0) - 1e-12)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    expect = [1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38, -0.0]
    assert np.array_equal(oracle.widen(bits), np.array(expect))


def test_physical_block_permutation_leaves_output_bitwise_unchanged():
    """Relabel every physical block by a permutation pi: K'[pi(p)] = K[p] and
    table' = pi(table).  The logical view, hence the output, is identical
    (aicassindra.com 'The block table: logical to physical mapping')."""
    case = synth.decode_case("c3s")
    cfg = case["cfg"]
    b = cfg["block_size"]
    rng = np.random.default_rng(7)
    nb = case["num_blocks"]
    bm = oracle.BlockManagerModel(nb, b, case["free_order"])
    kp = synth.nan_fill((nb, b, cfg["num_kv_heads"], cfg["head_dim"]), "bf16")
    vp = kp.copy()
    for s, L in enumerate(case["lengths"]):
        slots, _ = bm.append(s, int(L))
        o = case["offsets"]
        oracle.reshape_and_cache(kp, vp, case["keys"][o[s]:o[s + 1]], case["values"][o[s]:o[s + 1]], np.array(slots))
    maxb = max(len(bm.table(s)) for s in range(len(case["lengths"])))
    tables = np.zeros((len(case["lengths"]), maxb), np.int32)
    for s in range(len(case["lengths"])):
        t = bm.table(s)
        tables[s, :len(t)] = t
    pi = rng.permutation(nb)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[pi] = kp
    vp2[pi] = vp
    sub = [0, 3, 7]
    a = oracle.decode_attention(case["q"], kp, vp, tables, case["lengths"], case["scale"], seqs=sub)
    b2 = oracle.decode_attention(case["q"], kp2, vp2, pi[tables].astype(np.int32), case["lengths"], case["scale"], seqs=sub)
    assert np.array_equal(a, b2)


def test_slot_address_matches_printed_tables():
    """Widget table r2 = [9..13] at B=4: token 10 is in logical block 2, offset 2
    -> physical block 11 -> flat slot 46; token 0 of r3 -> block 14 -> slot 56."""
    w = GOLDEN["widget_tables"]
    assert oracle.slot_address(w["tables"][2], 10, w["block_size"]) == 46
    assert oracle.slot_address(w["tables"][3], 0, w["block_size"]) == 56
    assert oracle.slot_address(w["tables"][0], 16, w["block_size"]) == 16


def test_reshape_and_cache_round_trips_through_the_table():
    """Writing each token at its slot and reading the logical view back through
    the table returns the tokens in order; untouched slots keep their bytes."""
    rng = np.random.default_rng(8)
    bm = oracle.BlockManagerModel(20, 4, rng.permutation(20))
    keys = synth.byte_pattern((13, 2, 8), "bf16", 1)
    values = synth.byte_pattern((13, 2, 8), "bf16", 2)
    kp = synth.byte_pattern((20, 4, 2, 8), "bf16", 3)
    vp = synth.byte_pattern((20, 4, 2, 8), "bf16", 4)
    k0, v0 = kp.copy(), vp.copy()
    slots, _ = bm.append(0, 13)
    oracle.reshape_and_cache(kp, vp, keys, values, np.array(slots))
    table = bm.table(0)
    assert np.array_equal(oracle.gather_logical(kp, table, 13, 4), keys)
    assert np.array_equal(oracle.gather_logical(vp, table, 13, 4), values)
    written = np.zeros(80, bool)
    written[slots] = True
    assert np.array_equal(kp.reshape(80, 2, 8)[~written], k0.reshape(80, 2, 8)[~written])
    assert np.array_equal(vp.reshape(80, 2, 8)[~written], v0.reshape(80, 2, 8)[~written])


def test_reshape_and_cache_skips_negative_slots():
    kp = synth.byte_pattern((2, 4, 1, 8), "f32", 5)
    vp = synth.byte_pattern((2, 4, 1, 8), "f32", 6)
    k0 = kp.copy()
    oracle.reshape_and_cache(kp, vp, np.zeros((2, 1, 8), np.float32), np.zeros((2, 1, 8), np.float32), np.array([-1, 5]))
    assert np.array_equal(kp.view(np.uint32)[1, 1], np.zeros((1, 8), np.uint32))
    kp.reshape(8, 1, 8)[5] = k0.reshape(8, 1, 8)[5]
    assert np.array_equal(kp.view(np.uint32), k0.view(np.uint32))


def test_copy_blocks_copies_whole_blocks_only():
    kp = synth.byte_pattern((6, 4, 2, 8), "bf16", 9)
    vp = synth.byte_pattern((6, 4, 2, 8), "bf16", 10)
    k0, v0 = kp.copy(), vp.copy()
    oracle.copy_blocks(kp, vp, np.array([[1, 4], [2, 0]]))
    assert np.array_equal(kp[4], k0[1]) and np.array_equal(vp[4], v0[1])
    assert np.array_equal(kp[0], k0[2]) and np.array_equal(vp[0], v0[2])
    for b in (1, 2, 3, 5):
        assert np.array_equal(kp[b], k0[b]) and np.array_equal(vp[b], v0[b])
    with pytest.raises(ValueError):
        oracle.copy_blocks(kp, vp, np.array([[1, 4], [4, 5]]))
