"""pa_decode_plan_advance and plan reuse in pa_bm_prepare_decode_step (CPU).

Between decode steps every sequence grows by one token (S06
"Implementation" passes the length per call; mercemay.com "Blocks, tables,
and the indirection": a new block only every B tokens), so a plan can be
carried forward instead of rebuilt: new lengths in every job record, and the
last piece of each sequence that gained a tile one tile longer.  These tests
check that an advanced plan covers exactly the new lengths with the same
records and merge rows, that every case it cannot follow is refused with the
plan unchanged, and that the step preparation's reuse gives plans that cover
each step's lengths and rebuilds after the configured number of steps."""
import numpy as np
import pytest

import paged_kv_cache_115_amd as pk


def _coverage(plan, lens, hkv):
    """Every tile of every (sequence, head block) once; jobs carry the length."""
    hb_n = -(-hkv // 4)
    seen = {}
    for j in plan.jobs().tolist():
        seq, t0, cnt, hb, part, nparts, rb, L = j
        assert L == lens[seq] and cnt >= 1
        for t in range(t0, t0 + cnt):
            key = (seq, hb & 0xFFFF, t)
            assert key not in seen
            seen[key] = (part, nparts, rb)
    for s, L in enumerate(lens):
        for hb in range(hb_n):
            for t in range(-(-int(L) // 16)):
                assert (s, hb, t) in seen
    assert len(seen) == sum(-(-int(L) // 16) for L in lens) * hb_n
    return seen


def _parts(plan):
    return sorted((j[0], j[3], j[4], j[5], j[6]) for j in plan.jobs().tolist())


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("sched", [pk.SCHEDULE_LPT, pk.SCHEDULE_CHUNKS])
def test_advance_covers_new_lengths(seed, sched):
    rng = np.random.default_rng(700 + seed)
    lens = rng.integers(1, 900, size=int(rng.integers(5, 80))).astype(np.int32)
    lens[rng.random(len(lens)) < 0.1] = 0
    hkv = int(rng.choice([4, 8, 13]))
    nwg = int(rng.integers(3, 300))
    plan = pk.decode_plan(lens, hkv, nwg, 0, schedule=sched)
    plan.set_first_blocks(np.zeros((len(lens), 64), np.int32), 16)
    merges = plan.merges().copy()
    records, jobs = plan.num_records, plan.num_jobs
    parts0 = _parts(plan)
    for k in range(1, 40):
        new = np.where(lens > 0, lens + k, 0).astype(np.int32)
        assert plan.advance(new)
        _coverage(plan, new, hkv)
        plan.check_lens(new)
        # records, merge rows, job count and piece numbering stay
        assert np.array_equal(plan.merges(), merges) and plan.num_records == records and plan.num_jobs == jobs
        assert _parts(plan) == parts0
        assert plan.info.num_tiles == sum(int(j[2]) for j in plan.jobs().tolist())
        assert plan.info.max_job_tiles == max(int(j[2]) for j in plan.jobs().tolist())
        assert plan.info.max_context_len == int(new.max())
        assert plan.info.flags & pk.PA_DECODE_FIRST_BLOCKS == 0 and plan.info.first_block_size == 0


def test_advance_refuses_what_it_cannot_follow():
    lens = np.array([16, 17, 40, 0, 100], np.int32)
    plan = pk.decode_plan(lens, 8, 4, 2, schedule=pk.SCHEDULE_LPT)
    before = plan.blob.copy()
    info = bytes(plan.info)
    cases = [
        np.array([16, 17, 40, 0, 133], np.int32),   # +3 tiles
        np.array([16, 17, 40, 1, 100], np.int32),   # empty -> non-empty
        np.array([16, 17, 16, 0, 100], np.int32),   # 40 (3 tiles) -> 16 (1 tile)
        np.array([16, 17, 40, 0, 0], np.int32),     # 100 -> 0
    ]
    for new in cases:
        assert not plan.advance(new)
        assert np.array_equal(plan.blob, before) and bytes(plan.info) == info
    # a longer job than allowed: sequence 1 (17 tokens) is one 2-tile piece,
    # and 33 tokens would make it 3 tiles
    assert not plan.advance(np.array([16, 33, 40, 0, 100], np.int32), max_job_tiles=2)
    assert np.array_equal(plan.blob, before)
    assert plan.advance(np.array([16, 33, 40, 0, 100], np.int32))
    assert plan.advance(np.array([16, 33, 40, 0, 100], np.int32))   # the same lengths again: nothing to do
    # same tiles, other lengths: follows
    assert plan.advance(np.array([1, 48, 33, 0, 97], np.int32))
    with pytest.raises(pk.PaError):
        plan.advance(np.array([1, 2, 3], np.int32))
    with pytest.raises(pk.PaError):
        plan.advance(np.array([1, 48, -1, 0, 97], np.int32))
    # prefix plans are rebuilt, never advanced
    pre = pk.decode_plan_prefix([300] * 4, 8, 32, [0] * 4, [200] * 4, num_workgroups=8)
    assert pre.num_groups > 0 and not pre.advance(np.array([301] * 4, np.int32))


def test_advance_extends_last_piece_only():
    """A sequence crossing into a new tile extends, per head block, the job
    holding its last tile; the others keep their tiles."""
    lens = np.array([64, 200], np.int32)       # 4 and 13 tiles
    plan = pk.decode_plan(lens, 8, 6, 5, schedule=pk.SCHEDULE_LPT)
    old = {(j[0], j[3], j[1]): j[2] for j in plan.jobs().tolist()}
    assert plan.advance(np.array([65, 201], np.int32))
    new = {(j[0], j[3], j[1]): j[2] for j in plan.jobs().tolist()}
    assert old.keys() == new.keys()
    for (s, hb, t0), cnt in old.items():
        last = t0 + cnt == (4 if s == 0 else 13)
        assert new[(s, hb, t0)] == cnt + (1 if last and s == 0 else 0)


def _manager(lens, b=16, seed=4):
    rng = np.random.default_rng(seed)
    nb = int(sum(-(-int(L) // b) for L in lens)) + 4 * len(lens) + 64
    bm = pk.BlockManager(nb, b, rng.permutation(nb).astype(np.int32))
    for s, L in enumerate(lens):
        bm.append(s, int(L))
    return bm


@pytest.mark.parametrize("reuse", [0, 1, 5])
def test_prepare_step_with_plan_reuse(reuse):
    """With reuse, each step's plan covers that step's lengths; after `reuse`
    advances the next step builds afresh, which equals pa_decode_plan_schedule
    on the same lengths byte for byte."""
    lens0 = np.random.default_rng(12).integers(1, 300, 40).astype(np.int32)
    bm = _manager(lens0)
    bm.set_plan_reuse(reuse)
    seqs = np.arange(len(lens0))
    buf = np.zeros(1 << 22, np.uint8)
    buf = buf[(-buf.ctypes.data) % 256:]
    for k in range(1, 14):
        lay, plan = bm.prepare_decode_step(seqs, 64, 8, buf, 24, pk.SCHEDULE_LPT, True)
        lens = lens0 + k
        assert np.array_equal(buf[lay.lens_at:lay.lens_at + 4 * len(seqs)].view(np.int32), lens)
        _coverage(plan, lens, 8)
        plan.check_lens(lens)
        assert plan.info.flags & pk.PA_DECODE_FIRST_BLOCKS
        built = reuse == 0 or (k - 1) % (reuse + 1) == 0
        if built:
            fresh = pk.decode_plan(lens, 8, 24, 0, schedule=pk.SCHEDULE_LPT)
            fresh_jobs = fresh.blob[:fresh.info.merges_at]
            assert np.array_equal(plan.blob[:plan.info.merges_at], fresh_jobs)
    # another batch rebuilds
    lay, plan = bm.prepare_decode_step(seqs[:-1], 64, 8, buf, 24, pk.SCHEDULE_LPT, True)
    _coverage(plan, lens0[:-1] + 14, 8)
    with pytest.raises(pk.PaError):
        bm.set_plan_reuse(-1)
