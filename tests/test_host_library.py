"""CPU tests of the product library: it loads, exports every declared symbol,
its host block manager agrees with the Python model operation by operation,
and its argument checks reject bad calls before anything reaches a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import paged_kv_cache_115_amd as pk
from paged_kv_cache_115_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(pa_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 18
    for name in names:
        assert hasattr(_lib.lib, name), name
        assert name in _lib.SIGNATURES, f"{name} has no ctypes signature"


def test_widget_tables_through_the_library():
    bm = pk.BlockManager(64, 4)
    for r, L in enumerate([17, 16, 18, 8, 17, 10]):
        bm.append(r, L)
    assert [bm.table(r).tolist() for r in range(6)] == [
        [0, 1, 2, 3, 4], [5, 6, 7, 8], [9, 10, 11, 12, 13], [14, 15], [16, 17, 18, 19, 20], [21, 22, 23]]
    bm.check()


def _compare(bm: pk.BlockManager, model: oracle.BlockManagerModel, live):
    for s in live:
        assert bm.table(s).tolist() == model.table(s)
        assert bm.length(s) == model.length(s)
    for b in range(model.num_blocks):
        assert bm.refcount(b) == model.refcount[b]
    st, ms = bm.stats(), model.stats()
    for k in ms:
        assert st[k] == ms[k], k


@pytest.mark.parametrize("seed", range(12))
def test_block_manager_matches_model_on_random_operations(seed):
    rng = np.random.default_rng(seed)
    b = int(rng.choice([1, 4, 8, 16, 32]))
    nb = int(rng.integers(6, 90))
    order = rng.permutation(nb) if seed % 2 else None
    bm = pk.BlockManager(nb, b, order)
    model = oracle.BlockManagerModel(nb, b, order)
    live, nxt = [], 0
    for _ in range(250):
        op = int(rng.integers(0, 5))
        if op == 0 or not live:
            args = ("append", nxt, int(rng.integers(0, 3 * b)))
        elif op == 1:
            args = ("append", int(rng.choice(live)), int(rng.integers(0, 2 * b)))
        elif op == 2:
            args = ("fork", int(rng.choice(live)), nxt)
        elif op == 3:
            k = int(rng.integers(1, len(live) + 1))
            args = ("step", list(rng.choice(live, size=k, replace=False)))
        else:
            args = ("free", int(rng.choice(live)))
        if args[0] == "append":
            try:
                ms, mc = model.append(args[1], args[2])
                m_ok = True
            except oracle.OutOfBlocks:
                m_ok = False
            try:
                ps, pc = bm.append(args[1], args[2])
                p_ok = True
            except pk.PaError as e:
                assert e.status == -3
                p_ok = False
            assert m_ok == p_ok
            if m_ok:
                assert ps.tolist() == ms and [tuple(x) for x in pc.tolist()] == mc
                if args[1] not in live:
                    live.append(args[1])
                    nxt += 1
        elif args[0] == "fork":
            model.fork(args[1], args[2])
            bm.fork(args[1], args[2])
            live.append(args[2])
            nxt += 1
        elif args[0] == "step":
            try:
                ms, mc = model.append_step(args[1])
                m_ok = True
            except oracle.OutOfBlocks:
                m_ok = False
            try:
                ps, pc = bm.append_step(args[1])
                p_ok = True
            except pk.PaError:
                p_ok = False
            assert m_ok == p_ok
            if m_ok:
                assert ps.tolist() == ms and [tuple(x) for x in pc.tolist()] == mc
        else:
            model.free_seq(args[1])
            bm.free(args[1])
            live.remove(args[1])
        bm.check()
        _compare(bm, model, live)


def _compare_swaps(bm: pk.BlockManager, model: oracle.BlockManagerModel, live):
    _compare(bm, model, live)
    for s in live:
        assert bm.is_swapped(s) == model.is_swapped(s)
    for b in range(model.num_host_blocks):
        assert bm.host_refcount(b) == model.host_refcount[b]
    assert bm.host_refcount(model.num_host_blocks) == -1


@pytest.mark.parametrize("seed", range(10))
def test_block_manager_swaps_match_model(seed):
    """Appends, forks, frees and swaps in both directions, operation by
    operation: same pairs, tables, counts and failures as the model."""
    rng = np.random.default_rng(100 + seed)
    b = int(rng.choice([1, 4, 8, 16]))
    nb = int(rng.integers(8, 60))
    nh = int(rng.integers(0, 50))
    order = rng.permutation(nb) if seed % 2 else None
    bm = pk.BlockManager(nb, b, order)
    model = oracle.BlockManagerModel(nb, b, order)
    bm.set_host_blocks(nh)
    model.set_host_blocks(nh)
    live, nxt = [], 0
    for _ in range(250):
        resident = [s for s in live if not model.is_swapped(s)]
        swapped = [s for s in live if model.is_swapped(s)]
        op = int(rng.integers(0, 6))
        if op == 0 or not live:
            n = int(rng.integers(0, 3 * b))
            m_ok = p_ok = True
            try:
                ms, mc = model.append(nxt, n)
            except oracle.OutOfBlocks:
                m_ok = False
            try:
                ps, pc = bm.append(nxt, n)
            except pk.PaError:
                p_ok = False
            assert m_ok == p_ok
            if m_ok:
                assert ps.tolist() == ms and [tuple(x) for x in pc.tolist()] == mc
                live.append(nxt)
                nxt += 1
        elif op == 1 and resident:
            parent = int(rng.choice(resident))
            model.fork(parent, nxt)
            bm.fork(parent, nxt)
            live.append(nxt)
            nxt += 1
        elif op in (2, 3) and (resident if op == 2 else swapped):
            src = resident if op == 2 else swapped
            k = int(rng.integers(1, len(src) + 1))
            pick = [int(x) for x in rng.choice(src, size=k, replace=False)]
            m_fn, p_fn = (model.swap_out, bm.swap_out) if op == 2 else (model.swap_in, bm.swap_in)
            try:
                mp = m_fn(pick)
                m_ok = True
            except oracle.OutOfBlocks:
                m_ok = False
            try:
                pp = p_fn(pick)
                p_ok = True
            except pk.PaError as e:
                assert e.status == -3
                p_ok = False
            assert m_ok == p_ok
            if m_ok:
                assert [tuple(x) for x in pp.tolist()] == mp
        elif op == 4 and resident:
            s = int(rng.choice(resident))
            n = int(rng.integers(0, 2 * b))
            m_ok = p_ok = True
            try:
                model.append(s, n)
            except oracle.OutOfBlocks:
                m_ok = False
            try:
                bm.append(s, n)
            except pk.PaError:
                p_ok = False
            assert m_ok == p_ok
        elif op == 5:
            s = int(rng.choice(live))
            model.free_seq(s)
            bm.free(s)
            live.remove(s)
        bm.check()
        model.check()
        _compare_swaps(bm, model, live)


def _compare_cache(bm: pk.BlockManager, model: oracle.BlockManagerModel, live):
    _compare_swaps(bm, model, live)
    for b in range(model.num_blocks):
        assert bm.is_cached(b) == model.is_cached(b), b


@pytest.mark.parametrize("seed", range(10))
def test_prefix_cache_matches_model(seed):
    """Prompts drawn from a small vocabulary after one of a few system
    prompts (so that blocks repeat), plus appends, forks, swaps and frees:
    same slots, reuse counts, tables, counts, cache membership and failures
    as the model, operation by operation."""
    rng = np.random.default_rng(200 + seed)
    b = int(rng.choice([1, 2, 4, 8, 16]))
    nb = int(rng.integers(6, 70))
    order = rng.permutation(nb) if seed % 2 else None
    bm = pk.BlockManager(nb, b, order)
    model = oracle.BlockManagerModel(nb, b, order)
    bm.enable_prefix_cache()
    model.enable_prefix_cache()
    nh = int(rng.integers(0, 40))
    bm.set_host_blocks(nh)
    model.set_host_blocks(nh)
    vocab = int(rng.integers(2, 5))
    systems = [list(rng.integers(0, vocab, size=int(rng.integers(0, 4 * b + 2)))) for _ in range(3)]
    live, nxt = [], 0
    for _ in range(300):
        resident = [s for s in live if not model.is_swapped(s)]
        swapped = [s for s in live if model.is_swapped(s)]
        op = int(rng.integers(0, 8))
        if op <= 2 or not live:
            prompt = systems[int(rng.integers(0, 3))] + list(rng.integers(0, vocab, size=int(rng.integers(0, 3 * b))))
            m_ok = p_ok = True
            try:
                ms, mc = model.append_prompt(nxt, prompt)
            except oracle.OutOfBlocks:
                m_ok = False
            try:
                ps, pc = bm.append_prompt(nxt, prompt)
            except pk.PaError as e:
                assert e.status == -3
                p_ok = False
            assert m_ok == p_ok
            if m_ok:
                assert ps.tolist() == ms and pc == mc
                live.append(nxt)
                nxt += 1
        elif op == 3 and resident:
            s = int(rng.choice(resident))
            n = int(rng.integers(0, 2 * b))
            m_ok = p_ok = True
            try:
                ms, mc = model.append(s, n)
            except oracle.OutOfBlocks:
                m_ok = False
            try:
                ps, pc = bm.append(s, n)
            except pk.PaError:
                p_ok = False
            assert m_ok == p_ok
            if m_ok:
                assert ps.tolist() == ms and [tuple(x) for x in pc.tolist()] == mc
        elif op == 4 and resident:
            parent = int(rng.choice(resident))
            model.fork(parent, nxt)
            bm.fork(parent, nxt)
            live.append(nxt)
            nxt += 1
        elif op == 5 and (resident or swapped):
            out = bool(resident) and (not swapped or rng.random() < 0.5)
            pick = [int(rng.choice(resident if out else swapped))]
            m_fn, p_fn = (model.swap_out, bm.swap_out) if out else (model.swap_in, bm.swap_in)
            m_ok = p_ok = True
            try:
                mp = m_fn(pick)
            except oracle.OutOfBlocks:
                m_ok = False
            try:
                pp = p_fn(pick)
            except pk.PaError as e:
                assert e.status == -3
                p_ok = False
            assert m_ok == p_ok
            if m_ok:
                assert [tuple(x) for x in pp.tolist()] == mp
        elif op >= 6 and live:
            s = int(rng.choice(live))
            model.free_seq(s)
            bm.free(s)
            live.remove(s)
        bm.check()
        model.check()
        _compare_cache(bm, model, live)
    assert model.stats()["prefix_hit_tokens"] > 0


def test_prefix_cache_errors_through_the_library():
    bm = pk.BlockManager(8, 4)
    with pytest.raises(pk.PaError) as e:
        bm.append_prompt(0, [1, 2])               # cache off
    assert e.value.status == -1
    bm.append(0, 1)
    with pytest.raises(pk.PaError) as e:
        bm.enable_prefix_cache()                  # a sequence exists
    assert e.value.status == -1
    bm.free(0)
    bm.enable_prefix_cache()
    assert bm.append_prompt(0, [1, 2, 3, 4, 5])[1] == 0
    with pytest.raises(pk.PaError) as e:
        bm.append_prompt(0, [1, 2])               # sequence exists
    assert e.value.status == -1
    slots, cached = bm.append_prompt(1, [1, 2, 3, 4, 6])
    assert cached == 4 and slots.tolist()[:4] == [-1] * 4
    assert bm.append_prompt(2, [])[1] == 0 and bm.length(2) == 0
    assert bm.is_cached(0) and not bm.is_cached(1) and lib_cached(bm, 8) == -1
    bm.check()


def lib_cached(bm, block):
    return _lib.lib.pa_bm_cached(bm._h, block)


def test_block_manager_swap_errors():
    bm = pk.BlockManager(8, 4)
    bm.set_host_blocks(2)
    bm.append(0, 9)
    with pytest.raises(pk.PaError) as e:
        bm.swap_out([0])                  # three blocks, two host blocks
    assert e.value.status == -3 and not bm.is_swapped(0)
    bm.set_host_blocks(4)
    with pytest.raises(pk.PaError) as e:
        bm.swap_out([0, 0])
    assert e.value.status == -1
    with pytest.raises(pk.PaError) as e:
        bm.swap_out([5])
    assert e.value.status == -4
    with pytest.raises(pk.PaError) as e:
        bm.swap_in([0])                   # resident
    assert e.value.status == -1
    assert bm.swap_out([0]).tolist() == [[0, 0], [1, 1], [2, 2]]
    for call in (lambda: bm.append(0, 1), lambda: bm.append_step([0]), lambda: bm.fork(0, 1),
                 lambda: bm.export([0], 4), lambda: bm.prefix_groups([0]), lambda: bm.set_host_blocks(8)):
        with pytest.raises(pk.PaError) as e:
            call()
        assert e.value.status == -1
    assert bm.table(0).tolist() == [0, 1, 2] and bm.length(0) == 9
    # Too small a pair buffer changes nothing.
    seqs = np.array([0], dtype=np.int64)
    pairs = np.zeros((2, 2), dtype=np.int32)
    n = ctypes.c_int32(0)
    st = _lib.lib.pa_bm_swap_in(bm._h, seqs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1,
                                pairs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2, ctypes.byref(n))
    assert st == -1 and bm.is_swapped(0)
    bm.free(0)
    assert bm.stats()["free_host_blocks"] == 4 and bm.stats()["num_seqs"] == 0
    bm.check()
    with pytest.raises(KeyError):
        bm.is_swapped(0)


def test_block_manager_errors():
    with pytest.raises(pk.PaError):
        pk.BlockManager(0, 16)
    with pytest.raises(pk.PaError):
        pk.BlockManager(4, 16, [0, 1, 1, 2])
    bm = pk.BlockManager(4, 4)
    with pytest.raises(pk.PaError) as e:
        bm.fork(7, 8)
    assert e.value.status == -4
    bm.append(1, 3)
    with pytest.raises(pk.PaError) as e:
        bm.fork(1, 1)
    assert e.value.status == -1
    with pytest.raises(pk.PaError) as e:
        bm.append_step([1, 1])
    assert e.value.status == -1
    bm.free(99)           # unknown: no-op
    with pytest.raises(pk.PaError) as e:
        bm.append(2, 100)
    assert e.value.status == -3 and bm.stats()["alloc_failures"] == 1
    with pytest.raises(KeyError):
        bm.table(5)
    assert bm.refcount(-1) == -1 and bm.refcount(4) == -1
    tables, lens = bm.export([1], 4)
    assert tables.tolist() == [[0, 0, 0, 0]] and lens.tolist() == [3]
    with pytest.raises(pk.PaError):
        bm.export([1, 42], 4)


def _plan_model(lens, hkv, nwg, cap):
    """Independent statement of the schedule pa_decode_plan documents:
    (sequence, head block) tile streams in alternating length order, laid end
    to end and cut into nwg chunks of equal cost (tokens + 4 per stream) at
    tile boundaries by the tile midpoint; consecutive tiles of a stream in a
    chunk form jobs of at most cap tiles.  Returns (jobs per workgroup,
    merge rows, records)."""
    lens = [int(x) for x in lens]
    hb = -(-hkv // 4)
    cap = cap or 64
    live = sorted([s for s in range(len(lens)) if lens[s] > 0], key=lambda s: -lens[s])
    order = []
    while live:
        order.append(live.pop(0))
        if live:
            order.append(live.pop())
    total = sum((lens[s] + 4) * hb for s in order)
    tiles = sum(-(-lens[s] // 16) * hb for s in order)
    nwg = max(1, min(nwg, tiles))
    cum, records = 0, 0
    wg_jobs = [[] for _ in range(nwg)]
    streams = {}
    for s in order:
        for h in range(hb):
            pcs = []
            for t in range(-(-lens[s] // 16)):
                c = min(16, lens[s] - 16 * t) + (4 if t == 0 else 0)
                w = min(nwg - 1, ((2 * cum + c) * nwg) // (2 * total))
                cum += c
                if not pcs or pcs[-1][0] != w or pcs[-1][2] >= cap:
                    pcs.append([w, t, 0])
                pcs[-1][2] += 1
            base = -1
            if len(pcs) > 1:
                base = records
                records += len(pcs) * min(4, hkv - 4 * h)
            for p, (w, t0, cnt) in enumerate(pcs):
                wg_jobs[w].append((s, t0, cnt, h, p if len(pcs) > 1 else 0, len(pcs), base))
            streams[(s, h)] = (len(pcs), base)
    merges = []
    for s in range(len(lens)):
        if lens[s] == 0:
            merges += [(s, g, 0, -1) for g in range(hkv)]
            continue
        for h in range(hb):
            n, base = streams[(s, h)]
            if n > 1:
                merges += [(s, g, n, base + (g - 4 * h) * n) for g in range(4 * h, min(hkv, 4 * h + 4))]
    return wg_jobs, merges, records


def _lpt_model(lens, hkv, nwg, cap):
    """Independent statement of the largest-pieces-first schedule: every
    sequence cut into near-equal pieces of at most cap tiles (cap 0: twice
    the average tiles per workgroup, clamped to [4, 64]), one job per (piece, head
    block); jobs by size, largest first (ties in generation order), each to
    the least-loaded pair of workgroups {b, b + nwg/2} for an even grid, or
    the least-loaded workgroup for an odd one (ties: the one that reached that
    load first, initially by index), and within a pair to the lighter member
    (ties: b), after which each pair's jobs are re-split by modelled end time;
    a workgroup runs its jobs smallest first.  Returns (jobs per workgroup,
    merge rows, records)."""
    import heapq
    lens = [int(x) for x in lens]
    hb = -(-hkv // 4)
    total = sum(-(-L // 16) * hb for L in lens)
    cap = cap or min(64, max(4, -(-2 * total // nwg)))
    jobs, merges, records = [], [], 0
    for s, L in enumerate(lens):
        tiles = -(-L // 16)
        if tiles == 0:
            merges += [(s, g, 0, -1) for g in range(hkv)]
            continue
        parts = -(-tiles // cap)
        base = records if parts > 1 else -1
        if parts > 1:
            merges += [(s, g, parts, records + g * parts) for g in range(hkv)]
            records += parts * hkv
        t0 = 0
        for p in range(parts):
            cnt = tiles // parts + (1 if p < tiles % parts else 0)
            for h in range(hb):
                jobs.append((s, t0, cnt, h, p if parts > 1 else 0, parts, base + 4 * h * parts if base >= 0 else -1))
            t0 += cnt
    nwg = max(1, min(nwg, len(jobs)))
    order = sorted(range(len(jobs)), key=lambda i: (-jobs[i][2], i))
    # An even grid balances pairs {b, b + nwg/2} (the workgroups that share a
    # compute unit), then splits each pair's jobs to its lighter member.
    bins = nwg // 2 if nwg % 2 == 0 else nwg
    heap = [(0, b, b) for b in range(bins)]
    arrival = bins
    wg_jobs = [[] for _ in range(nwg)]
    wg_load = [0] * nwg
    for i in order:
        load, _, b = heapq.heappop(heap)
        w = b + bins if nwg % 2 == 0 and wg_load[b + bins] < wg_load[b] else b
        wg_jobs[w].append(i)
        wg_load[w] += jobs[i][2]
        heapq.heappush(heap, (load + jobs[i][2], arrival, b))
        arrival += 1
    if nwg % 2 == 0:
        # Each pair's jobs (up to 8) are then split over its two workgroups to
        # minimise the modelled end time: b (dispatched first) streams 0.51
        # tiles/us while both run, b + nwg/2 0.32, either alone 0.75, and each
        # job costs 0.5 us; every subset for b, in mask order, first minimum.
        for b in range(bins):
            pj = sorted(wg_jobs[b] + wg_jobs[b + bins])
            if not 2 <= len(pj) <= 8:
                continue
            best, best_m = float("inf"), 0
            for m in range(1 << len(pj)):
                older = float(sum(jobs[i][2] for k, i in enumerate(pj) if m >> k & 1))
                younger = float(sum(jobs[i][2] for k, i in enumerate(pj) if not m >> k & 1))
                jo = bin(m).count("1")
                jy = len(pj) - jo
                t_o = older * (1.0 / 0.51) + 0.5 * jo
                t_y = younger * (1.0 / 0.32) + 0.5 * jy
                if t_o <= t_y:
                    e = t_o + max(0.0, younger - 0.32 * max(0.0, t_o - 0.5 * jy)) * (1.0 / 0.75)
                else:
                    e = t_y + max(0.0, older - 0.51 * max(0.0, t_y - 0.5 * jo)) * (1.0 / 0.75)
                if e < best:
                    best, best_m = e, m
            wg_jobs[b] = [i for k, i in enumerate(pj) if best_m >> k & 1]
            wg_jobs[b + bins] = [i for k, i in enumerate(pj) if not best_m >> k & 1]
    # Each workgroup runs its jobs smallest first, ties in generation order.
    return [[jobs[i] for i in sorted(l, key=lambda i: (jobs[i][2], i))] for l in wg_jobs], merges, records


def _plan_lists(plan):
    tab = plan.job_table()
    return [[tuple(j[:7]) for j in tab[:, b].tolist() if j[2] > 0] for b in range(tab.shape[1])]


def test_decode_plan_small_example():
    """Lengths 0, 5, 600, 1000 (0, 1, 38, 63 tiles), 8 KV heads (two head
    blocks), 6 workgroups.  Stream order 1000, 5, 600; costs 1004, 9, 604 per
    head block, 3234 in all, 539 per workgroup."""
    plan = pk.decode_plan([0, 5, 600, 1000], 8, num_workgroups=6, schedule=pk.SCHEDULE_CHUNKS)
    assert plan.schedule == pk.SCHEDULE_CHUNKS
    lists = _plan_lists(plan)
    # Worked by hand: a tile of cost c ending at cumulative cost e goes to
    # workgroup floor((e - c/2) / 539); e.g. the 1000-token stream of head
    # block 0 has midpoints 10, 28, 44, ... so its tiles 0..32 go to
    # workgroup 0 (midpoint 524) and 33..62 to workgroup 1.
    assert lists == [
        [(3, 0, 33, 0, 0, 2, 0)],
        [(3, 33, 30, 0, 1, 2, 0), (3, 0, 4, 1, 0, 3, 8)],
        [(3, 4, 34, 1, 1, 3, 8)],
        [(3, 38, 25, 1, 2, 3, 8), (1, 0, 1, 0, 0, 1, -1), (1, 0, 1, 1, 0, 1, -1), (2, 0, 8, 0, 0, 2, 20)],
        [(2, 8, 30, 0, 1, 2, 20), (2, 0, 4, 1, 0, 2, 28)],
        [(2, 4, 34, 1, 1, 2, 28)]]
    assert lists == _plan_model([0, 5, 600, 1000], 8, 6, 0)[0]
    tiles = [sum(j[2] for j in l) for l in lists]
    assert sum(tiles) == 2 * (63 + 1 + 38)
    merges = [tuple(m) for m in plan.merges().tolist()]
    assert merges[:8] == [(0, g, 0, -1) for g in range(8)]
    assert merges[8:12] == [(2, g, 2, 20 + 2 * g) for g in range(4)]
    assert merges[12:16] == [(2, g, 2, 28 + 2 * (g - 4)) for g in range(4, 8)]
    assert merges[16:20] == [(3, g, 2, 2 * g) for g in range(4)]
    assert merges[20:] == [(3, g, 3, 8 + 3 * (g - 4)) for g in range(4, 8)]
    assert plan.num_records == 36
    assert pk.decode_workspace_bytes(plan, 32, 128) >= 36 * 4 * 130 * 4


def test_decode_plan_small_example_lpt():
    """The same batch under the largest-pieces-first schedule: 204 job tiles
    over 6 workgroups, cap 34: 600 tokens (38 tiles) -> pieces 19 + 19,
    1000 tokens (63 tiles) -> 32 + 31, times two head blocks; the 5-token
    sequence is one tile per head block."""
    plan = pk.decode_plan([0, 5, 600, 1000], 8, num_workgroups=6, max_piece_tiles=34, schedule=pk.SCHEDULE_LPT)
    assert plan.schedule == pk.SCHEDULE_LPT
    assert (plan.num_workgroups, plan.num_jobs, plan.num_merges, plan.num_records) == (6, 10, 24, 32)
    jobs = sorted(map(tuple, plan.jobs()[:, :7].tolist()))
    assert jobs == sorted([
        (1, 0, 1, 0, 0, 1, -1), (1, 0, 1, 1, 0, 1, -1),
        (2, 0, 19, 0, 0, 2, 0), (2, 0, 19, 1, 0, 2, 8), (2, 19, 19, 0, 1, 2, 0), (2, 19, 19, 1, 1, 2, 8),
        (3, 0, 32, 0, 0, 2, 16), (3, 0, 32, 1, 0, 2, 24), (3, 32, 31, 0, 1, 2, 16), (3, 32, 31, 1, 1, 2, 24)])
    loads = sorted(int(plan.job_table()[:, w, 2].sum()) for w in range(6))
    assert loads == [31, 32, 32, 33, 38, 38]
    # Placement by compute-unit pairs {0, 3}, {1, 4}, {2, 5}: 32 -> pair 0,
    # 32 -> pair 1, 31 and 31 -> pair 2, the four 19-tile jobs alternate over
    # pairs 0 and 1, the two 1-tile jobs go to pair 2.  Each pair is then split
    # by modelled end time, the first-dispatched member taking the larger
    # share: pairs 0 and 1 give 19 + 19 to b and 32 to b + 3, pair 2 gives
    # 31 + 1 + 1 to 2 and 31 to 5.
    per_wg = [int(plan.job_table()[:, w, 2].sum()) for w in range(6)]
    assert per_wg == [38, 38, 33, 32, 32, 31]
    merges = [tuple(m) for m in plan.merges().tolist()]
    assert merges == ([(0, g, 0, -1) for g in range(8)] + [(2, g, 2, 2 * g) for g in range(8)] +
                      [(3, g, 2, 16 + 2 * g) for g in range(8)])
    assert lists_equal_model(plan, [0, 5, 600, 1000], 8, 6, 34, _lpt_model)
    # The default piece is twice the 34-tile average, clamped to 64: the
    # 38- and 63-tile sequences stay whole.
    whole = pk.decode_plan([0, 5, 600, 1000], 8, num_workgroups=6, schedule=pk.SCHEDULE_LPT)
    assert (whole.num_jobs, whole.num_records) == (6, 0)
    assert lists_equal_model(whole, [0, 5, 600, 1000], 8, 6, 0, _lpt_model)
    auto = pk.decode_plan([0, 5, 600, 1000], 8, num_workgroups=6)
    assert auto.schedule in (pk.SCHEDULE_CHUNKS, pk.SCHEDULE_LPT)
    with pytest.raises(pk.PaError):
        pk.decode_plan([1], 8, num_workgroups=6, schedule=2)


def lists_equal_model(plan, lens, hkv, nwg, cap, model):
    wg_jobs, merges, records = model(lens, hkv, nwg, cap)
    return (_plan_lists(plan) == wg_jobs and [tuple(m) for m in plan.merges().tolist()] == merges
            and plan.num_records == records)


@pytest.mark.parametrize("seed", range(12))
def test_decode_plan_matches_model(seed):
    rng = np.random.default_rng(100 + seed)
    lens = rng.integers(0, 3000, size=int(rng.integers(1, 60)))
    lens[rng.random(len(lens)) < 0.2] = int(rng.integers(0, 40))
    hkv = int(rng.choice([1, 3, 4, 8, 13]))
    nwg = int(rng.integers(1, 900))
    cap = int(rng.choice([0, 1, 5, 64]))
    for sched, model in ((pk.SCHEDULE_CHUNKS, _plan_model), (pk.SCHEDULE_LPT, _lpt_model)):
        p = pk.decode_plan(lens, hkv, num_workgroups=nwg, max_piece_tiles=cap, schedule=sched)
        assert p.schedule == sched
        if p.num_jobs:
            assert lists_equal_model(p, lens, hkv, nwg, cap, model)
    plan = pk.decode_plan(lens, hkv, num_workgroups=nwg, max_piece_tiles=cap)
    model = _plan_model if plan.schedule == 0 else _lpt_model
    wg_jobs, merges, records = model(lens, hkv, nwg, cap)
    if plan.num_jobs == 0:
        assert sum(map(len, wg_jobs)) == 0
    else:
        assert _plan_lists(plan) == wg_jobs
    assert [tuple(m) for m in plan.merges().tolist()] == merges
    assert plan.num_records == records


@pytest.mark.parametrize("seed", range(6))
def test_decode_plan_covers_every_tile_once(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 3000, size=int(rng.integers(1, 60)))
    hkv = int(rng.choice([1, 3, 4, 8, 13]))
    nwg = int(rng.integers(1, 900))
    cap = int(rng.choice([0, 1, 5, 64]))
    plan = pk.decode_plan(lens, hkv, num_workgroups=nwg, max_piece_tiles=cap)
    jobs = plan.jobs()
    hb = -(-hkv // 4)
    covered = {}
    for seq, t0, cnt, blk, part, parts, base, _ in jobs.tolist():
        assert 1 <= cnt <= 64 and (cap == 0 or cnt <= cap)
        for t in range(t0, t0 + cnt):
            key = (seq, blk, t)
            assert key not in covered
            covered[key] = (part, parts, base)
    for s, L in enumerate(lens):
        tiles = -(-int(L) // 16)
        for blk in range(hb):
            for t in range(tiles):
                assert (s, blk, t) in covered
    assert len(covered) == sum(-(-int(L) // 16) for L in lens) * hb
    assert plan.info.num_tiles == len(covered) == int(jobs[:, 2].sum())
    assert plan.num_workgroups <= nwg and len(jobs) == plan.num_jobs
    if plan.num_jobs:
        tab = plan.job_table()
        filled = tab[:, :, 2] > 0
        # each workgroup's jobs fill a prefix of its column
        assert np.all(filled[1:] <= filled[:-1])
        # cost of a workgroup (tokens + 4 per stream start) within the costs
        # of half its first and half its last tile (<= 20 each) of the mean
        cost = np.zeros(plan.num_workgroups)
        for b in range(plan.num_workgroups):
            for seq, t0, cnt, *_ in tab[:, b].tolist():
                if cnt > 0:
                    cost[b] += sum(min(16, int(lens[seq]) - 16 * t) + (4 if t == 0 else 0) for t in range(t0, t0 + cnt))
        mean = cost.sum() / plan.num_workgroups
        if plan.schedule == 0:
            assert cost.max() <= mean + 20 + 1e-9
            if mean >= 40:
                assert cost.min() >= mean - 20 - 1e-9
        else:
            loads = tab[:, :, 2].sum(axis=0)
            assert loads.max() <= np.ceil(loads.sum() / plan.num_workgroups) + jobs[:, 2].max()


def test_decode_plan_errors():
    with pytest.raises(pk.PaError):
        pk.decode_plan([1, -2], 8, num_workgroups=4)
    with pytest.raises(pk.PaError):
        pk.decode_plan([1, 2], 8, num_workgroups=4, max_piece_tiles=65)
    with pytest.raises(pk.PaError):
        pk.decode_plan([1, 2], 0, num_workgroups=4)
    with pytest.raises(pk.PaError):
        pk.decode_plan([1, 2], 8, num_workgroups=0)
    empty = pk.decode_plan([], 8, num_workgroups=4)
    assert (empty.num_jobs, empty.num_merges, empty.num_records) == (0, 0, 0)


class _Pool(ctypes.Structure):
    _fields_ = _lib.PaKvPool._fields_


def _pool(dtype=1, b=16, d=128, hkv=8, k=0x10000, v=0x20000):
    return _lib.PaKvPool(k, v, 100, b, hkv, d, dtype)


@pytest.mark.parametrize("pool,status", [
    (_pool(dtype=5), -2), (_pool(b=12), -2), (_pool(d=64), -2), (_pool(dtype=0, d=96), -2),
    (_pool(k=0), -1), (_pool(k=0x10004), -1)])
def test_abi_rejects_bad_pools_without_launching(pool, status):
    dummy = ctypes.c_void_p(0x30000)
    st = _lib.lib.pa_reshape_and_cache(ctypes.byref(pool), dummy, dummy, dummy, 4, None)
    assert st == status
    assert _lib.lib.pa_last_error()
    st = _lib.lib.pa_copy_blocks(ctypes.byref(pool), dummy, 1, None)
    assert st == status


def test_abi_rejects_bad_swap_arguments_without_launching():
    dev = _pool()
    L = _lib.lib

    def call(host=None, pairs=((0, 1),), direction=0, engine=0, n=None):
        arr = np.ascontiguousarray(np.array(pairs, dtype=np.int32).reshape(-1, 2))
        ptr = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if arr.size else None
        return L.pa_swap_blocks(ctypes.byref(dev), ctypes.byref(host or _pool(k=0x50000, v=0x60000)), ptr,
                                arr.shape[0] if n is None else n, direction, engine, None)

    assert call(pairs=(), n=0) == 0                          # no pairs: no-op, no HIP call
    assert call(host=_pool(b=8, k=0x50000, v=0x60000)) == -1  # block shape differs
    assert call(host=_pool(dtype=0, k=0x50000, v=0x60000)) == -1
    assert call(host=_pool(k=0)) == -1
    assert call(host=_pool(k=0x50004, v=0x60000)) == -1      # alignment
    assert call(direction=2) == -1
    assert call(engine=7) == -1
    assert call(n=-1) == -1
    assert call(pairs=((100, 0),)) == -1                     # source outside the device pool
    assert call(pairs=((0, 100),)) == -1                     # destination outside the host pool
    assert call(pairs=((0, 1), (2, 1))) == -1                # destination repeats
    assert call(pairs=((0, -1),), direction=1) == -1
    assert b"destination" in L.pa_last_error()
    dev_bad = _pool(b=12)
    assert L.pa_swap_blocks(ctypes.byref(dev_bad), ctypes.byref(_pool()), None, 0, 0, 0, None) == -2


@pytest.mark.parametrize("b", [8, 16, 32])
def test_first_tile_entries_match_the_tables(b):
    """pa_decode_plan_first_blocks writes, per job slot, the table entries
    of the job's tiles 0 and 1 (entry 2t and 2t + 1 at B = 8, t at B = 16,
    t / 2 at B = 32), 0 for an entry past the sequence's ceil(L / B) (never
    read), zeros for empty slots."""
    rng = np.random.default_rng(70 + b)
    lens = rng.integers(0, 400, size=37)
    maxb = int(max(-(-int(L) // b) for L in lens))
    tables = rng.integers(0, 5000, size=(37, maxb)).astype(np.int32)
    for sched, cap in ((pk.SCHEDULE_CHUNKS, 3), (pk.SCHEDULE_LPT, 0)):
        plan = pk.decode_plan(lens, 8, num_workgroups=13, max_piece_tiles=cap, schedule=sched)
        assert plan.info.flags == 0 and plan.info.first_block_size == 0
        assert plan.first_blocks().sum() == 0
        plan.set_first_blocks(tables, b)
        assert plan.info.flags & pk.PA_DECODE_FIRST_BLOCKS and plan.info.first_block_size == b
        tab, fb = plan.job_table(), plan.first_blocks()
        for k in range(tab.shape[0]):
            for w in range(tab.shape[1]):
                seq, t0, cnt = tab[k, w, :3]
                if cnt == 0:
                    assert fb[k, w].tolist() == [0, 0, 0, 0]
                    continue
                want = []
                for part in (0, 1):
                    for kk in (0, 1):
                        t = t0 + kk
                        e = 2 * t + part if b == 8 else (t // (b // 16) if part == 0 else None)
                        used = -(-int(lens[seq]) // b)
                        want.append(0 if e is None or e >= used else int(tables[seq, e]))
                assert fb[k, w].tolist() == want, (k, w)
    with pytest.raises(pk.PaError):
        plan.set_first_blocks(tables[:5], b)          # jobs name sequences past the rows given
    with pytest.raises(pk.PaError):
        plan.set_first_blocks(tables, 12)


def test_abi_rejects_bad_decode_arguments_without_launching():
    pool = _pool()
    p = ctypes.c_void_p(0x40000)
    L = _lib.lib
    plan = pk.decode_plan([100, 3000], 8, num_workgroups=4)
    assert plan.num_records > 0

    def call(info=None, **kw):
        args = dict(q=p, out=p, out_dtype=0, tables=p, maxb=400, lens=p, nseq=2, hq=32, scale=0.1, plan=p,
                    ws=None, wsb=0, nk=None, nv=None)
        args.update(kw)
        return L.pa_decode(ctypes.byref(pool), args["q"], args["out"], args["out_dtype"], args["tables"],
                           args["maxb"], args["lens"], args["nseq"], args["hq"], ctypes.c_float(args["scale"]),
                           args["nk"], args["nv"], args["plan"], ctypes.byref(info or plan.info), args["ws"],
                           args["wsb"], None)
    ws = dict(ws=ctypes.c_void_p(0x50000), wsb=1 << 30)
    assert call(hq=30, **ws) == -1                  # not a multiple of Hkv
    assert call(hq=8 * 17, **ws) == -2              # group of 17 > 16
    assert call(out_dtype=7, **ws) == -2
    assert call(q=None, **ws) == -1
    assert call(q=ctypes.c_void_p(0x40008), **ws) == -1   # misaligned
    assert call() == -1                             # workspace missing
    assert call(ws=ctypes.c_void_p(0x50000), wsb=16) == -1   # too small
    assert call(scale=float("inf"), **ws) == -1
    assert call(nk=p, **ws) == -1                   # new_key without new_value
    assert call(nk=ctypes.c_void_p(0x40008), nv=p, **ws) == -1   # misaligned new_key
    other = pk.decode_plan([100, 3000], 4, num_workgroups=4)
    assert call(info=other.info, **ws) == -1        # plan made for another head count
    bad = _lib.PaDecodePlanInfo.from_buffer_copy(plan.info)
    bad.jobs_at = 8
    assert call(info=bad, **ws) == -1               # inconsistent layout
    bad = _lib.PaDecodePlanInfo.from_buffer_copy(plan.info)
    bad.merges_at = 0
    assert call(info=bad, **ws) == -1               # merge list overlaps the job table
    flagged = _lib.PaDecodePlanInfo.from_buffer_copy(plan.info)
    flagged.flags = 4
    assert call(info=flagged, **ws) == -1           # unknown flag bit
    first = _lib.PaDecodePlanInfo.from_buffer_copy(plan.info)
    first.flags = pk.PA_DECODE_FIRST_BLOCKS
    first.first_block_size = 8
    assert call(info=first, **ws) == -1             # first-tile entries for another block size
    assert b"first-tile" in L.pa_last_error()
    for stage in (L.pa_decode_attention, L.pa_decode_merge_pieces):   # same checks on both stages
        assert stage(ctypes.byref(pool), p, p, 0, p, 400, p, 2, 30, ctypes.c_float(0.1), None, None, p,
                     ctypes.byref(plan.info), ws["ws"], ws["wsb"], None) == -1
        assert b"pa_decode_" in L.pa_last_error()
    empty = pk.decode_plan([], 8, num_workgroups=4)
    assert call(info=empty.info) == 0               # nothing to do: OK, no launch
    pool32 = _pool(dtype=0, d=64)
    assert L.pa_decode(ctypes.byref(pool32), p, p, 1, p, 400, p, 2, 8, ctypes.c_float(1.0), None, None, p,
                       ctypes.byref(plan.info), ws["ws"], ws["wsb"], None) == -2   # bf16 output, f32 pool


# ------------------------------------------------------------ prefix groups
def _forked_batch(b, prompts, samples, prefix, tails, order_seed=3):
    """Block manager holding `prompts` prompts of `prefix` tokens, each forked
    into `samples` sequences that then append their own tails (the first
    divergent token copies the shared partial block)."""
    rng = np.random.default_rng(order_seed)
    nb = prompts * (prefix // b + 2) + samples * prompts * (max(tails) // b + 3) + 8
    bm = pk.BlockManager(nb, b, rng.permutation(nb).astype(np.int32))
    for i in range(prompts):
        bm.append(1000 + i, prefix)
        for j in range(samples):
            bm.fork(1000 + i, i * samples + j)
        bm.free(1000 + i)
    seqs = np.arange(prompts * samples)
    bm.append_step(seqs)
    for s in seqs:
        if tails[s] > 1:
            bm.append(int(s), int(tails[s]) - 1)
    return bm, seqs


@pytest.mark.parametrize("b", [8, 16, 32])
def test_prefix_groups_of_forked_samples(b):
    """Samples of one prompt form one group sharing the prompt's full blocks
    (the partial block is copied at the fork); unrelated sequences are alone."""
    tails = np.array([5, 1, 30, 2, 7, 3, 9, 1])
    bm, seqs = _forked_batch(b, 2, 4, 100, tails)
    bm.append(77, 40)                       # an unrelated sequence
    batch = np.concatenate([seqs, [77]])
    group, tokens = bm.prefix_groups(batch)
    assert group.tolist() == [0, 0, 0, 0, 4, 4, 4, 4, -1]
    full = (100 // b) * b
    assert tokens.tolist() == [full] * 8 + [0]
    # The same from the exported tables: longest common run of leading blocks.
    tables, lens = bm.export(batch, 64)
    for g0 in (0, 4):
        rows = tables[g0:g0 + 4]
        nb = [min(-(-int(L) // b), 64) for L in lens[g0:g0 + 4]]
        c = 0
        while all(c < n for n in nb) and len({int(r[c]) for r in rows}) == 1:
            c += 1
        assert c * b == full


def test_prefix_plan_cache_policy():
    """Loads keep blocks in the caches only if a shared block is read by more
    than one job: a key group of more members than fit one group (G = 4: four
    members), or a group without a whole shared tile."""
    plan = pk.decode_plan_prefix([300] * 4, 8, 32, [0] * 4, [200] * 4, num_workgroups=8)
    assert plan.num_groups > 0 and plan.info.flags == 0            # one group of four: each block read once
    plan = pk.decode_plan_prefix([300] * 6, 8, 32, [0] * 6, [200] * 6, num_workgroups=8)
    assert plan.info.flags == pk.PA_DECODE_SHARED_KV              # six members: two groups read the prefix
    plan = pk.decode_plan_prefix([300] * 2, 8, 32, [0] * 2, [10] * 2, num_workgroups=8)
    assert plan.num_groups == 0 and plan.info.flags == pk.PA_DECODE_SHARED_KV   # under one tile: both read it
    plan = pk.decode_plan_prefix([300, 200], 8, 32, [-1, -1], [0, 0], num_workgroups=8)
    assert plan.info.flags == 0
    plan = pk.decode_plan_prefix([300] * 8, 8, 64, [0] * 4 + [4] * 4, [200] * 8, num_workgroups=8)
    assert plan.info.flags == pk.PA_DECODE_SHARED_KV              # G = 8: two members per group


def _check_prefix_plan(plan, lens, hkv, hq, group, tokens):
    """Structural invariants of a shared-prefix plan, per (sequence, KV head,
    tile): every tile of every sequence read by exactly one job, shared
    pieces numbered before each member's own pieces, records disjoint.  A
    wide job (PA_JOB_WIDE) reads one KV head for a set of up to four groups
    whose descriptors lie ceil(hkv / 4) apart."""
    G = hq // hkv
    cap = min(4, max(1, 16 // G))
    hb_n = -(-hkv // 4)
    tab = plan.job_table()
    jobs = [tuple(j) for b in range(tab.shape[1]) for j in tab[:, b].tolist() if j[2] > 0]
    groups = plan.groups()
    covered = {}
    own = {}
    wide_jobs = 0

    def cover(s, g, t0, cnt, what):
        for t in range(t0, t0 + cnt):
            assert (s, g, t) not in covered
            covered[(s, g, t)] = what

    for seq, t0, cnt, hbf, part, nparts, rb, L in jobs:
        shared = bool(hbf & pk.PA_JOB_SHARED)
        assert L == lens[seq] and 1 <= cnt <= 64
        if shared and hbf & pk.PA_JOB_WIDE:
            wide_jobs += 1
            g = hbf & 0xFFFF
            ngr, full, last = nparts & 0xFF, (nparts >> 8) & 0xFF, (nparts >> 16) & 0xFF
            assert 1 <= ngr <= 4 and 0 <= g < hkv
            for k in range(ngr):
                d = groups[rb + k * hb_n]
                n = int(d[0])
                assert n == (full if k < ngr - 1 else last) and 2 <= n <= cap and d[1] == g // 4
                assert k > 0 or d[2] == seq
                for m in range(n):
                    cover(int(d[2 + m]), g, t0, cnt, ("shared", part))
        elif shared:
            hb = hbf & 0xFFFF
            d = groups[rb]
            n = int(d[0])
            assert 2 <= n <= cap and d[1] == hb and d[2] == seq and nparts == n
            for m in range(n):
                for g in range(4 * hb, min(hkv, 4 * hb + 4)):
                    cover(int(d[2 + m]), g, t0, cnt, ("shared", part))
        else:
            hb = hbf & 0xFFFF
            for g in range(4 * hb, min(hkv, 4 * hb + 4)):
                cover(seq, g, t0, cnt, ("own", part))
            own.setdefault((seq, hb), []).append((part, nparts, rb))
    assert plan.info.wide_jobs == wide_jobs
    for s, L in enumerate(lens):
        for g in range(hkv):
            for t in range(-(-int(L) // 16)):
                assert (s, g, t) in covered
    # num_tiles counts the tiles read: a shared tile once for its whole group (or set)
    assert plan.info.num_tiles == sum(j[2] for j in jobs)
    # every group's members: shared pieces 0 .. k - 1 on every KV head of the
    # head block, own pieces k .. parts - 1, records consistent and disjoint
    used = set()
    for d in groups:
        n, hb = int(d[0]), int(d[1])
        for m in range(n):
            s, rb, np_ = int(d[2 + m]), int(d[6 + m]), int(d[10 + m])
            parts = sorted(own[(s, hb)])
            assert all(p[1] == np_ and p[2] == rb for p in parts)
            ks = None
            for g in range(4 * hb, min(hkv, 4 * hb + 4)):
                shared_parts = sorted({v[1] for k, v in covered.items() if k[0] == s and k[1] == g and v[0] == "shared"})
                assert shared_parts == list(range(len(shared_parts)))
                assert ks is None or ks == len(shared_parts)
                ks = len(shared_parts)
            assert [p[0] for p in parts] == list(range(ks, np_))
            for w in range(min(4, hkv - 4 * hb)):
                for p in range(np_):
                    r = rb + w * np_ + p
                    assert r not in used and 0 <= r < plan.num_records
                    used.add(r)
    merges = {(int(m[0]), int(m[1])): (int(m[2]), int(m[3])) for m in plan.merges()}
    for (s, hb), parts in own.items():
        np_, rb = parts[0][1], parts[0][2]
        for g in range(4 * hb, min(hkv, 4 * hb + 4)):
            if np_ > 1:
                assert merges[(s, g)] == (np_, rb + (g - 4 * hb) * np_)
            else:
                assert (s, g) not in merges


@pytest.mark.parametrize("b", [8, 16, 32])
def test_prefix_plan_structure(b):
    tails = np.array([5, 1, 30, 2, 7, 3, 9, 1, 60, 4])
    bm, seqs = _forked_batch(b, 2, 5, 300, tails)
    bm.append(77, 40)
    batch = np.concatenate([seqs, [77]])
    tables, lens = bm.export(batch, 64)
    group, tokens = bm.prefix_groups(batch)
    for hkv, hq, nwg in [(8, 32, 7), (8, 32, 512), (4, 32, 5), (3, 6, 9)]:
        plan = pk.decode_plan_prefix(lens, hkv, hq, group, tokens, num_workgroups=nwg)
        assert plan.num_groups > 0
        G = hq // hkv
        assert plan.group_size == min(4, 16 // G, 5)
        _check_prefix_plan(plan, lens, hkv, hq, group, tokens)
    # a shared part below one tile, or groups of one, plan no sharing
    none = pk.decode_plan_prefix(lens, 8, 32, group, np.minimum(tokens, 15), num_workgroups=8)
    assert none.num_groups == 0
    alone = pk.decode_plan_prefix(lens, 8, 32, np.arange(len(lens)), tokens, num_workgroups=8)
    assert alone.num_groups == 0
    with pytest.raises(pk.PaError):
        pk.decode_plan_prefix(lens, 8, 30, group, tokens, num_workgroups=8)


def _wide_batch(b=16, prompts=3, samples=20, prefix=1000, seed=5):
    rng = np.random.default_rng(seed)
    tails = rng.integers(1, 200, prompts * samples)
    bm, seqs = _forked_batch(b, prompts, samples, prefix, tails)
    tables, lens = bm.export(seqs, 128)
    group, tokens = bm.prefix_groups(seqs)
    return lens, group, tokens


@pytest.mark.parametrize("nwg", [512, 64, 72, 7])
def test_wide_prefix_plan_invariants(nwg):
    """Key groups of more members than one group holds (G = 4: 20 samples of
    a prompt make 5 groups of 4) keep every plan invariant, whatever the grid
    (die-aware placement on grids that are multiples of 8 and at least 64,
    the chunk schedule otherwise)."""
    lens, group, tokens = _wide_batch()
    for hkv, hq in [(8, 32), (4, 16), (8, 64), (3, 6)]:
        plan = pk.decode_plan_prefix(lens, hkv, hq, group, tokens, num_workgroups=nwg)
        assert plan.num_groups > 0 and plan.info.flags == pk.PA_DECODE_SHARED_KV
        _check_prefix_plan(plan, lens, hkv, hq, group, tokens)
        # The full grid reads each prefix in sets of groups, per KV head; a
        # grid that is not a multiple of the 8 dies never does.
        if nwg == 512:
            assert plan.info.wide_jobs > 0
        if nwg == 7:
            assert plan.info.wide_jobs == 0


def test_wide_sets_fall_back_when_cuts_differ():
    """A die holding more of a key group's head streams than workgroups cuts
    them unevenly; the four KV heads of a set's head block would then hold
    different numbers of shared pieces, which the per-head-block record
    layout cannot express, so the plan reads every group on its own."""
    rng = np.random.default_rng(5)
    bm, seqs = _forked_batch(16, 12, 20, 600, rng.integers(1, 200, 240))
    tables, lens = bm.export(seqs, 128)
    group, tokens = bm.prefix_groups(seqs)
    sets = pk.decode_plan_prefix(lens, 8, 32, group, tokens, num_workgroups=64)
    alone = pk.decode_plan_prefix(lens, 4, 16, group, tokens, num_workgroups=64)
    assert sets.info.wide_jobs > 0 and alone.info.wide_jobs == 0
    _check_prefix_plan(sets, lens, 8, 32, group, tokens)
    _check_prefix_plan(alone, lens, 4, 16, group, tokens)


def _placement(plan):
    """Per workgroup: its jobs in slot order as (shared, group descriptor, head
    block, tile_begin, tile_count, seq)."""
    tab = plan.job_table()
    out = []
    for b in range(tab.shape[1]):
        out.append([(bool(j[3] & pk.PA_JOB_SHARED), int(j[6]), int(j[3] & 0xFFFF), int(j[1]), int(j[2]), int(j[0]))
                    for j in tab[:, b].tolist() if j[2] > 0])
    return out


@pytest.mark.parametrize("nwg", [512, 64])
def test_wide_prefix_placement_meets_on_one_die(nwg):
    """The shared streams of one wide prefix (several groups of one key group,
    per head block) run on one die (workgroup b on die b mod 8), cut into the
    same tile ranges, one piece per workgroup; the first half of a die's
    workgroups run it before their other jobs, the second half after them;
    and the chunk walk tops every workgroup up to about the same cost."""
    lens, group, tokens = _wide_batch()
    hkv, hq = 8, 32
    plan = pk.decode_plan_prefix(lens, hkv, hq, group, tokens, num_workgroups=nwg)
    groups = plan.groups()
    place = _placement(plan)
    per_die = nwg // 8
    key_of = lambda d: int(group[int(groups[d][2])])
    sets = {}
    for b, jobs in enumerate(place):
        sh = [j for j in jobs if j[0]]
        for k, j in enumerate(jobs):
            if j[0]:
                sets.setdefault((key_of(j[1]), j[2]), []).append((b % 8, b, j[1], j[3], j[4]))
        if sh:
            # one shared piece per workgroup here; first half: first, second half: last
            assert len(sh) == 1
            i = b // 8
            pos = jobs.index(sh[0])
            assert pos == 0 if 2 * i < per_die else pos == len(jobs) - 1
    for (key, hb), pieces in sets.items():
        dies = {p[0] for p in pieces}
        assert len(dies) <= 2
        # the pieces of one die and set share their tile ranges
        for die in dies:
            ranges = {}
            for _, b, d, t0, cnt in pieces:
                if b % 8 == die:
                    ranges.setdefault(d, []).append((t0, cnt))
            shapes = {tuple(sorted(v)) for v in ranges.values()}
            assert len(shapes) == 1, shapes
    # cost balance: shared tile = 12, own token = 1 (+ the walk's stream charge)
    cost = np.array([sum(12 * j[4] if j[0] else min(int(lens[j[5]]), 16 * (j[3] + j[4])) - 16 * j[3]
                         for j in jobs) for jobs in place])
    assert cost.max() <= cost.mean() * 1.15 + 64, (cost.max(), cost.mean())
