"""CPU tests of pa_bm_prepare_decode_step: one call and one buffer for a
serving loop's host work per decode step.  It must equal, byte for byte, the
separate calls it replaces (pa_bm_append_step, the tables' used entries,
pa_decode_plan_schedule for the new lengths, pa_decode_plan_first_blocks),
and every refusal must leave the block manager unchanged."""
import numpy as np
import pytest

import paged_kv_cache_115_amd as pk


def _aligned(nbytes: int) -> np.ndarray:
    raw = np.zeros(nbytes + 256, dtype=np.uint8)
    off = (-raw.ctypes.data) % 256
    return raw[off:off + nbytes]


def _managers(b, seed):
    """Two identical block managers: a batch with forks (copy-on-write at the
    next append), an empty sequence and lengths at block edges."""
    rng = np.random.default_rng(seed)
    nb = 600
    order = rng.permutation(nb).astype(np.int32)
    out = []
    for _ in range(2):
        bm = pk.BlockManager(nb, b, order)
        lens = [0, 1, b - 1, b, b + 1, 3 * b + 5, 200, 37]
        for s, n in enumerate(lens):
            bm.append(s, n)
        bm.fork(6, 8)            # shares a partial block: the next append copies it
        bm.fork(3, 9)            # shares only full blocks
        out.append(bm)
    return out


@pytest.mark.parametrize("b", [8, 16, 32])
@pytest.mark.parametrize("schedule", [pk.SCHEDULE_AUTO, pk.SCHEDULE_CHUNKS, pk.SCHEDULE_LPT])
def test_prepare_step_equals_the_separate_calls(b, schedule):
    bm, ref = _managers(b, 40 + b)
    seqs = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 9], dtype=np.int64)
    maxb = 40
    buf = _aligned(1 << 20)
    buf[:] = 0xAB
    for step in range(3):
        lay, plan = bm.prepare_decode_step(seqs, maxb, 8, buf, num_workgroups=7, schedule=schedule)
        slots, cows = ref.append_step(seqs)
        tables, lens = ref.export(seqs, maxb)
        want = pk.decode_plan(lens, 8, num_workgroups=7, schedule=schedule).set_first_blocks(tables, b)
        assert np.array_equal(buf[lay.slots_at:lay.slots_at + 8 * len(seqs)].view(np.int64), slots)
        assert lay.n_cows == len(cows)
        assert np.array_equal(buf[lay.cows_at:lay.cows_at + 8 * lay.n_cows].view(np.int32).reshape(-1, 2), cows)
        assert np.array_equal(buf[lay.lens_at:lay.lens_at + 4 * len(seqs)].view(np.int32), lens)
        rows = buf[lay.tables_at:lay.tables_at + 4 * len(seqs) * maxb].view(np.int32).reshape(len(seqs), maxb)
        for i, L in enumerate(lens):
            n = -(-int(L) // b)
            assert np.array_equal(rows[i, :n], tables[i, :n])
        assert lay.plan.bytes == want.info.bytes and lay.bytes == lay.plan_at + lay.plan.bytes
        assert np.array_equal(plan.blob, want.blob), step
        for f in ("num_seqs", "max_context_len", "lens_digest", "num_jobs", "flags", "first_block_size"):
            assert getattr(plan.info, f) == getattr(want.info, f), f
        plan.check_lens(lens)
        bm.check()
    assert step == 2 and lay.n_cows == 0


def test_prepare_step_refusals_change_nothing():
    bm, _ = _managers(16, 3)
    seqs = np.arange(10, dtype=np.int64)
    before = [bm.length(int(s)) for s in seqs]
    with pytest.raises(pk.PaError):
        bm.prepare_decode_step(seqs, 20, 8, _aligned(1024), num_workgroups=7)          # buffer too small
    with pytest.raises(pk.PaError):
        bm.prepare_decode_step(np.array([0, 99]), 20, 8, _aligned(1 << 20), num_workgroups=7)   # unknown sequence
    with pytest.raises(pk.PaError):
        bm.prepare_decode_step(seqs, 12, 8, _aligned(1 << 20), num_workgroups=7)     # 200 + 1 tokens need 13 rows
    with pytest.raises(pk.PaError):
        bm.prepare_decode_step(seqs, 20, 8, _aligned(1 << 20)[1:], num_workgroups=7)  # misaligned
    assert [bm.length(int(s)) for s in seqs] == before
    bm.check()
    small = pk.BlockManager(4, 16)
    small.append(0, 64)                                                               # pool full
    with pytest.raises(pk.PaError) as e:
        small.prepare_decode_step([0], 8, 8, _aligned(1 << 16), num_workgroups=2)
    assert e.value.status == -3 and small.length(0) == 64
