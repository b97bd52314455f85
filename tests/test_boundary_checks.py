"""CPU tests of the decode boundary's consistency checks.

A decode plan is built on the host for one batch's context lengths, and
lengths grow by one every step, so a plan kept from another step, or made for
another batch, must be refused or made harmless.  The plan records the batch
size, its longest context and a digest of the lengths; pa_decode refuses a
plan made for another num_seqs or for tables too short for its longest
context before anything is launched; pa_decode_plan_check_lens and the
pa_validate_* calls check, on host copies, what only the device holds (slots,
copy pairs, table entries, lengths against the plan, appends into shared
blocks).  The pages' warning that a wrong block or count shows up as corrupted
attention scores rather than a crash (mercemay.com "Paged KV Cache Allocation
and the Block Table", "Sharing blocks between sequences") is why these exist.
Every test here runs without a GPU: the library rejects each call before any
HIP call."""
import ctypes
import types

import numpy as np
import pytest
import torch

import paged_kv_cache_115_amd as pk
from paged_kv_cache_115_amd import _lib

L = _lib.lib


def _pool(nb=100, b=16, hkv=8, d=128, dtype=1):
    return _lib.PaKvPool(0x10000, 0x20000, nb, b, hkv, d, dtype)


def _fake_pool(nb=100, b=16, hkv=8, d=128):
    """A stand-in for KvPool for the host-side checks (no device memory)."""
    k = torch.empty((nb, b, hkv, d), dtype=torch.bfloat16, device="meta")
    return types.SimpleNamespace(k=k, v=k, c=_pool(nb, b, hkv, d), block_size=b)


def test_plan_records_what_it_was_made_for():
    lens = np.array([5, 0, 300, 17], dtype=np.int32)
    plan = pk.decode_plan(lens, 8, num_workgroups=6)
    assert plan.info.num_seqs == 4
    assert plan.info.max_context_len == 300
    plan.check_lens(lens)
    with pytest.raises(pk.PaError, match="other context lengths"):
        plan.check_lens(lens + (lens > 0))          # the next step's lengths
    with pytest.raises(pk.PaError, match="4 sequences"):
        plan.check_lens(lens[:3])
    # Equal lengths give equal digests whatever the schedule; any change differs.
    other = pk.decode_plan(lens, 8, num_workgroups=9, schedule=pk.SCHEDULE_LPT)
    assert other.info.lens_digest == plan.info.lens_digest
    for i in range(4):
        bumped = lens.copy()
        bumped[i] += 1
        assert pk.decode_plan(bumped, 8, num_workgroups=6).info.lens_digest != plan.info.lens_digest
    prefix = pk.decode_plan_prefix(lens, 8, 32, [0, -1, 0, -1], [16, 0, 16, 0], num_workgroups=6)
    assert (prefix.info.num_seqs, prefix.info.max_context_len) == (4, 300)
    prefix.check_lens(lens)
    empty = pk.decode_plan([], 8, num_workgroups=4)
    assert empty.info.num_seqs == 0 and empty.info.max_context_len == 0
    empty.check_lens([])


def _decode_call(plan_info, nseq, maxb, pool=None):
    p = ctypes.c_void_p(0x40000)
    pool = pool or _pool()
    return L.pa_decode(ctypes.byref(pool), p, p, 0, p, maxb, p, nseq, 32, ctypes.c_float(0.1), None, None, p,
                       ctypes.byref(plan_info), ctypes.c_void_p(0x50000), 1 << 30, None)


def test_decode_refuses_a_plan_for_another_batch_before_launching():
    plan = pk.decode_plan([100, 3000], 8, num_workgroups=4)
    assert _decode_call(plan.info, 3, 400) == -1
    assert b"plan made for 2 sequences" in L.pa_last_error()
    assert _decode_call(plan.info, 1, 400) == -1
    for stage in (L.pa_decode_attention, L.pa_decode_merge_pieces):
        p = ctypes.c_void_p(0x40000)
        assert stage(ctypes.byref(_pool()), p, p, 0, p, 400, p, 3, 32, ctypes.c_float(0.1), None, None, p,
                     ctypes.byref(plan.info), ctypes.c_void_p(0x50000), 1 << 30, None) == -1


def test_decode_refuses_tables_too_short_for_the_plan():
    plan = pk.decode_plan([100, 3000], 8, num_workgroups=4)
    # 3000 tokens need 188 entries of 16 slots: 187 is one short.
    assert _decode_call(plan.info, 2, 187) == -1
    assert b"longest context" in L.pa_last_error()
    # With 32-slot blocks 94 entries cover 3008 tokens: the check passes and
    # the call then fails only on the dummy pointers' HIP launch, which this
    # test does not reach (a pool of another block size is checked instead).
    assert _decode_call(plan.info, 2, 93, pool=_pool(b=32)) == -1
    assert b"longest context" in L.pa_last_error()


def test_validate_slots():
    pool = _fake_pool(nb=4, b=16)               # 64 slots
    pk.validate_slots(pool, np.array([0, 63, -1, -1, 17], dtype=np.int64))   # negatives are padding
    pk.validate_slots(pool, np.zeros(0, dtype=np.int64))
    with pytest.raises(pk.PaError, match="slot 64"):
        pk.validate_slots(pool, np.array([3, 64], dtype=np.int64))
    with pytest.raises(pk.PaError, match="tokens 0 and 2 write the same slot 5"):
        pk.validate_slots(pool, np.array([5, 6, 5], dtype=np.int64))


def test_validate_copy_pairs():
    pool = _fake_pool(nb=10)
    pk.validate_copy_pairs(pool, np.array([[0, 1], [2, 3], [0, 4]], dtype=np.int32))   # a source may repeat
    pk.validate_copy_pairs(pool, np.zeros((0, 2), dtype=np.int32))
    with pytest.raises(pk.PaError, match="outside the pool"):
        pk.validate_copy_pairs(pool, np.array([[0, 10]], dtype=np.int32))
    with pytest.raises(pk.PaError, match="outside the pool"):
        pk.validate_copy_pairs(pool, np.array([[-1, 3]], dtype=np.int32))
    with pytest.raises(pk.PaError, match="destination of two pairs"):
        pk.validate_copy_pairs(pool, np.array([[0, 3], [1, 3]], dtype=np.int32))
    with pytest.raises(pk.PaError, match="both a source and a destination"):
        pk.validate_copy_pairs(pool, np.array([[0, 3], [3, 4]], dtype=np.int32))


def _batch(b=16):
    """Three sequences from the block manager: 40, 1 and 33 tokens."""
    bm = pk.BlockManager(32, b, np.random.default_rng(5).permutation(32).astype(np.int32))
    for s, n in enumerate([40, 1, 33]):
        bm.append(s, n)
    tables, lens = bm.export(np.arange(3), 4)
    return bm, tables, lens


def test_validate_decode_accepts_the_block_managers_batch():
    bm, tables, lens = _batch()
    pool = _fake_pool(nb=32)
    for sched in (pk.SCHEDULE_CHUNKS, pk.SCHEDULE_LPT):
        plan = pk.decode_plan(lens, 8, num_workgroups=5, max_piece_tiles=1, schedule=sched)
        pk.validate_decode(pool, tables, lens, plan)
        pk.validate_decode(pool, tables, lens, plan, fused_append=True)


def test_validate_decode_refuses_a_stale_plan():
    bm, tables, lens = _batch()
    pool = _fake_pool(nb=32)
    stale = pk.decode_plan(lens, 8, num_workgroups=5)
    bm.append_step(np.arange(3))                # the next step: every length + 1
    tables2, lens2 = bm.export(np.arange(3), 4)
    with pytest.raises(pk.PaError, match="other context lengths"):
        pk.validate_decode(pool, tables2, lens2, stale)
    pk.validate_decode(pool, tables2, lens2, pk.decode_plan(lens2, 8, num_workgroups=5))


def test_validate_decode_refuses_a_job_with_another_length():
    """A plan whose digest matches but whose job records were altered."""
    bm, tables, lens = _batch()
    pool = _fake_pool(nb=32)
    plan = pk.decode_plan(lens, 8, num_workgroups=5)
    tab = plan.job_table()
    k, w = np.argwhere(tab[:, :, 2] > 0)[0]
    tab[k, w, 7] += 16
    with pytest.raises(pk.PaError, match="was planned for"):
        pk.validate_decode(pool, tables, lens, plan)
    tab[k, w, 7] -= 16
    tab[k, w, 0] = 7                            # a sequence past the batch
    with pytest.raises(pk.PaError, match="names sequence 7"):
        pk.validate_decode(pool, tables, lens, plan)


def test_validate_decode_refuses_bad_table_entries_and_lengths():
    bm, tables, lens = _batch()
    pool = _fake_pool(nb=32)
    plan = pk.decode_plan(lens, 8, num_workgroups=5)
    bad = tables.copy()
    bad[2, 2] = 32                              # sequence 2 (33 tokens) uses entries 0..2
    with pytest.raises(pk.PaError, match="logical block 2 names block 32"):
        pk.validate_decode(pool, bad, lens, plan)
    bad[2, 2] = -1
    with pytest.raises(pk.PaError, match="names block -1"):
        pk.validate_decode(pool, bad, lens, plan)
    unused = tables.copy()
    unused[1, 1:] = 999                         # entries past ceil(L / B) are never read
    pk.validate_decode(pool, unused, lens, plan)
    with pytest.raises(pk.PaError, match="table row holds 2 blocks"):
        pk.validate_decode(pool, tables[:, :2], lens, plan)   # 40 tokens need 3 entries


def test_validate_decode_refuses_an_append_into_a_shared_block():
    """Forked sequences name the same partial block until copy-on-write gives
    the writer its own; a fused append before that would write into the
    block the sibling reads."""
    bm = pk.BlockManager(16, 16)
    bm.append(0, 20)
    bm.fork(0, 1)
    tables, lens = bm.export(np.arange(2), 2)
    pool = _fake_pool(nb=16)
    plan = pk.decode_plan(lens, 8, num_workgroups=3)
    pk.validate_decode(pool, tables, lens, plan)              # reading shared blocks is fine
    with pytest.raises(pk.PaError, match="another sequence also names"):
        pk.validate_decode(pool, tables, lens, plan, fused_append=True)
    bm.append_step(np.arange(2))                              # copy-on-write separates them
    tables, lens = bm.export(np.arange(2), 2)
    pk.validate_decode(pool, tables, lens, pk.decode_plan(lens, 8, num_workgroups=3), fused_append=True)


@pytest.mark.parametrize("what", ["head_dim", "tables", "lens", "out", "new_key"])
def test_decode_binding_checks_shapes_before_anything(what):
    """The C ABI has no head_dim for q and no row counts for the tables and
    lengths: the binding checks them against the pool before any call."""
    pool = _fake_pool(nb=32, d=128)
    S, hq = 3, 32
    meta = dict(device="meta")
    q = torch.empty((S, hq, 64 if what == "head_dim" else 128), dtype=torch.bfloat16, **meta)
    tables = torch.empty((S + (what == "tables"), 4), dtype=torch.int32, **meta)
    lens = torch.empty((S - (what == "lens"),), dtype=torch.int32, **meta)
    out = torch.empty((S, hq, 127 if what == "out" else 128), dtype=torch.float32, **meta)
    nk = torch.empty((S, 8 if what != "new_key" else 4, 128), dtype=torch.bfloat16, **meta)
    plan = pk.decode_plan([1, 2, 3], 8, num_workgroups=3)
    with pytest.raises(ValueError):
        pk.decode(pool, q, tables, lens, 0.1, plan, None, out=out, new_key=nk, new_value=nk)


def test_debug_mode_switch():
    pk.set_debug(True)
    try:
        assert pk._debug
    finally:
        pk.set_debug(False)
    assert not pk._debug
