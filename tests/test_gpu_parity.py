"""GPU parity: the HIP path against the float64 oracle on identical seeded
inputs.  Cache kernels bit-exact; attention within the stated tolerances;
invariances bitwise.

A schedule is (persistent workgroups, longest piece in tiles): None/0 is the
library default for the device; a few workgroups give long job lists per
workgroup; tiny pieces cut every sequence and exercise the merge launch."""
import numpy as np
import pytest
import torch

import oracle
import synth

from flows import (assert_close, bits, cascade_decode, gpu_decode, oracle_decode_step, oracle_prefix,
                   plan_and_workspace, product_decode_step, product_prefix, to_dev, to_host)

pytestmark = pytest.mark.gpu

DEFAULT = (None, 0)
FEW_WG = (3, 0)
TINY_PIECES = (None, 1)
SMALL_PIECES = (7, 3)


@pytest.fixture(scope="module")
def pk():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import paged_kv_cache_115_amd as m
    return m


def log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------ cache kernels
@pytest.mark.parametrize("dt,b,hkv,d", [("f32", 16, 4, 64), ("bf16", 16, 8, 128), ("bf16", 8, 8, 128),
                                        ("bf16", 32, 2, 128), ("f32", 32, 3, 128), ("bf16", 1, 8, 128),
                                        ("bf16", 4, 8, 128), ("f32", 2, 4, 64)])
def test_reshape_and_cache_bit_exact(pk, dt, b, hkv, d):
    log(f"reshape_and_cache dt={dt} B={b} Hkv={hkv} D={d}")
    rng = np.random.default_rng(21)
    nb = max(61, 2 * 400 // b)
    shape = (nb, b, hkv, d)
    kp = synth.byte_pattern(shape, dt, 1)
    vp = synth.byte_pattern(shape, dt, 2)
    n = 300
    slots = rng.choice(nb * b, size=n, replace=False).astype(np.int64)
    slots[::7] = -1
    key = synth.byte_pattern((n, hkv, d), dt, 3)
    val = synth.byte_pattern((n, hkv, d), dt, 4)
    kd, vd = to_dev(kp), to_dev(vp)
    pool = pk.KvPool(kd, vd)
    pk.reshape_and_cache(pool, to_dev(key), to_dev(val), to_dev(slots))
    oracle.reshape_and_cache(kp, vp, key, val, slots)
    assert np.array_equal(bits(to_host(kd)), bits(kp))
    assert np.array_equal(bits(to_host(vd)), bits(vp))


@pytest.mark.parametrize("dt,b,hkv,d", [("bf16", 16, 8, 128), ("bf16", 32, 8, 128), ("f32", 8, 4, 64),
                                        ("bf16", 2, 8, 128), ("f32", 1, 4, 64)])
def test_copy_blocks_bit_exact(pk, dt, b, hkv, d):
    log(f"copy_blocks dt={dt} B={b}")
    rng = np.random.default_rng(22)
    nb = 64
    shape = (nb, b, hkv, d)
    kp = synth.byte_pattern(shape, dt, 5)
    vp = synth.byte_pattern(shape, dt, 6)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:20], perm[20:40]], axis=1).astype(np.int32)
    kd, vd = to_dev(kp), to_dev(vp)
    pool = pk.KvPool(kd, vd)
    pk.copy_blocks(pool, to_dev(pairs))
    pk.copy_blocks(pool, to_dev(np.zeros((0, 2), np.int32)))     # empty: no-op
    oracle.copy_blocks(kp, vp, pairs)
    assert np.array_equal(bits(to_host(kd)), bits(kp))
    assert np.array_equal(bits(to_host(vd)), bits(vp))


# ------------------------------------------------------------ decode parity
DECODE_CASES = [("c1", DEFAULT), ("c1", TINY_PIECES), ("c1", FEW_WG), ("c2s", DEFAULT), ("c2s", SMALL_PIECES),
                ("c3s", DEFAULT), ("c3s", FEW_WG), ("c3s", TINY_PIECES), ("c3s", SMALL_PIECES),
                ("c4s", DEFAULT), ("c4s", SMALL_PIECES)]


@pytest.mark.parametrize("name,schedule", DECODE_CASES)
def test_decode_step_matches_oracle(pk, name, schedule):
    log(f"decode step {name} schedule={schedule}")
    case = synth.decode_case(name)
    dt = case["cfg"]["dtype"]
    got = product_decode_step(pk, case, schedule)
    ref = oracle_decode_step(case)
    assert np.array_equal(got["tables"], ref["tables"])
    assert [list(x) for x in got["pre_slots"]] == [list(x) for x in ref["pre_slots"]]
    assert got["new_slots"] == ref["new_slots"]
    assert np.array_equal(bits(got["kpool"]), bits(ref["kpool"]))
    assert np.array_equal(bits(got["vpool"]), bits(ref["vpool"]))
    stats = assert_close(got["out"], ref["out"], dt, f"{name}/{schedule}")
    log(f"  max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g}")


FIRST_CASES = [("c1", DEFAULT), ("c2s", DEFAULT), ("c2s", SMALL_PIECES), ("c3s", DEFAULT), ("c3s", TINY_PIECES),
               ("c3s", FEW_WG), ("c4s", SMALL_PIECES)]


@pytest.mark.parametrize("name,schedule", FIRST_CASES)
def test_first_tile_entries_in_the_plan_change_no_bit(pk, name, schedule):
    """A plan carrying the jobs' first-tile table entries
    (pa_decode_plan_first_blocks) gives bitwise the output of the same plan
    without them, separate and fused append alike."""
    log(f"first-tile entries {name} schedule={schedule}")
    case = synth.decode_case(name)
    got = product_decode_step(pk, case, schedule)
    args = (pk, got["pool"], got["q_dev"], got["tables"], got["lens"], case["scale"], schedule)
    base = to_host(gpu_decode(*args))
    first = to_host(gpu_decode(*args, first_blocks=True))
    assert np.array_equal(bits(base), bits(got["out"])) and np.array_equal(bits(first), bits(base))


@pytest.mark.parametrize("b", [8, 16, 32])
def test_first_tile_entries_at_edge_lengths_and_fused(pk, b):
    """Lengths that put the first tiles at block and tile edges (1, B-1, B,
    B+1, 16, 17, 32), with the append fused into the launch: pools and output
    equal, bit for bit, with and without the plan's first-tile entries."""
    log(f"first-tile entries edge lengths B={b}")
    for fused in (False, True):
        runs = []
        for first in (False, True):
            case = _edge_case([1, b - 1, b, b + 1, 16, 17, 32, 3 * b + 5], b)
            runs.append(product_decode_step(pk, case, FEW_WG, fused=fused, first_blocks=first))
        assert np.array_equal(bits(runs[0]["out"]), bits(runs[1]["out"]))
        assert np.array_equal(bits(runs[0]["kpool"]), bits(runs[1]["kpool"]))
        assert np.array_equal(bits(runs[0]["vpool"]), bits(runs[1]["vpool"]))


FUSED_CASES = [("c1", DEFAULT), ("c1", TINY_PIECES), ("c2s", SMALL_PIECES), ("c3s", DEFAULT), ("c3s", TINY_PIECES),
               ("c3s", FEW_WG), ("c4s", SMALL_PIECES)]


@pytest.mark.parametrize("name,schedule", FUSED_CASES)
def test_fused_append_equals_separate_cache_write(pk, name, schedule):
    """pa_decode with new_key/new_value stores the appended token into its
    slot while attending: pools byte-identical to the oracle's (untouched
    slots still NaN), output bitwise equal to pa_reshape_and_cache followed
    by pa_decode."""
    log(f"fused append {name} schedule={schedule}")
    case = synth.decode_case(name)
    fused = product_decode_step(pk, case, schedule, fused=True)
    split = product_decode_step(pk, case, schedule)
    ref = oracle_decode_step(case)
    assert np.array_equal(bits(fused["kpool"]), bits(ref["kpool"]))
    assert np.array_equal(bits(fused["vpool"]), bits(ref["vpool"]))
    assert np.array_equal(bits(fused["out"]), bits(split["out"]))
    assert_close(fused["out"], ref["out"], case["cfg"]["dtype"], f"fused {name}/{schedule}")


@pytest.mark.parametrize("long_context", [False, True])
@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32])
def test_fused_append_edge_lengths(pk, b, long_context):
    """The appended token at every position of a tile and of a block, in
    empty, one-token and full-table contexts, for each block size.  These
    contexts average 18 tiles, so the library loads every tile through
    per-lane addresses; one added 12,000-token context lifts the average to
    about 50, where only the appended token's tile is loaded that way."""
    lens = [0, 1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 0, 255, 256, 257, 1023, 1024, 1025, 2100]
    if long_context:
        lens.append(12000)
    case = _edge_case(lens, b)
    ref = oracle_decode_step(case)
    for schedule in (DEFAULT, TINY_PIECES, (5, 64)):
        log(f"fused edge lengths B={b} long={long_context} schedule={schedule}")
        got = product_decode_step(pk, case, schedule, fused=True)
        assert np.array_equal(bits(got["kpool"]), bits(ref["kpool"]))
        assert np.array_equal(bits(got["vpool"]), bits(ref["vpool"]))
        assert_close(got["out"], ref["out"], "bf16", f"fused edge/B{b}/{schedule}")


def test_decode_is_deterministic_and_schedule_independent_within_tolerance(pk):
    case = synth.decode_case("c3s")
    a = product_decode_step(pk, case, SMALL_PIECES)
    again = gpu_decode(pk, a["pool"], a["q_dev"], a["tables"], a["lens"], case["scale"], SMALL_PIECES)
    assert np.array_equal(to_host(again), a["out"])
    b = product_decode_step(pk, case, DEFAULT)
    assert np.abs(a["out"] - b["out"]).max() < 2e-3


def test_attention_then_merge_stages_equal_pa_decode(pk):
    """pa_decode_attention followed by pa_decode_merge_pieces on one stream
    writes bitwise what pa_decode writes (cut, uncut and empty sequences)."""
    case = synth.decode_case("c3s")
    a = product_decode_step(pk, case, SMALL_PIECES)
    lens = a["lens"].copy()
    lens[1] = 0          # an empty sequence: only the merge launch writes it
    plan, plan_dev, ws = plan_and_workspace(pk, lens, a["pool"].k.shape[2], a["q_dev"].shape[1],
                                            a["pool"].k.shape[3], *SMALL_PIECES)
    assert plan.num_records > 0 and plan.num_merges > 0
    args = (a["pool"], a["q_dev"], to_dev(a["tables"]), to_dev(lens), case["scale"], plan, plan_dev, ws)
    whole = torch.full(tuple(a["q_dev"].shape), float("nan"), device="cuda")
    pk.decode(*args, out=whole)
    staged = torch.full(tuple(a["q_dev"].shape), float("nan"), device="cuda")
    pk.decode(*args, out=staged, stage="attention")
    pk.decode(*args, out=staged, stage="merge")
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(whole)), bits(to_host(staged)))
    assert np.all(to_host(staged)[1] == 0)


def test_captured_graph_replays_match_eager_calls(pk):
    """A step captured as a HIP graph (the appended tokens' cache write, the
    attention launch, the merge launch), replayed several times with eager
    work and synchronisations between replays, writes what eager calls do."""
    case = synth.decode_case("c3s")
    a = product_decode_step(pk, case, SMALL_PIECES)
    off, lens_h = case["offsets"], a["lens"]
    rows = np.array([off[s + 1] - 1 for s in range(len(lens_h))])
    new_k, new_v = to_dev(case["keys"][rows]), to_dev(case["values"][rows])
    slots = to_dev(np.array(a["new_slots"], dtype=np.int64))
    pool, q = a["pool"], a["q_dev"]
    plan, plan_dev, ws = plan_and_workspace(pk, lens_h, pool.k.shape[2], q.shape[1], pool.k.shape[3], *SMALL_PIECES)
    assert plan.num_merges > 0
    tables, lens = to_dev(a["tables"]), to_dev(lens_h)
    eager = torch.full(tuple(q.shape), float("nan"), device="cuda")
    pk.reshape_and_cache(pool, new_k, new_v, slots)
    pk.decode(pool, q, tables, lens, case["scale"], plan, plan_dev, ws, out=eager)
    torch.cuda.synchronize()
    out = torch.full(tuple(q.shape), float("nan"), device="cuda")
    cap = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        pk.reshape_and_cache(pool, new_k, new_v, slots, cap)
        pk.decode(pool, q, tables, lens, case["scale"], plan, plan_dev, ws, out=out, stream=cap)
    for _ in range(4):
        out.fill_(float("nan"))
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(to_host(out)), bits(to_host(eager)))


def test_physical_block_permutation_is_bitwise_invariant(pk):
    """Same logical content through two different free-list orders."""
    case = synth.decode_case("c3s")
    a = product_decode_step(pk, case, SMALL_PIECES)
    case2 = dict(case)
    case2["free_order"] = np.random.default_rng(99).permutation(case["num_blocks"]).astype(np.int32)
    b = product_decode_step(pk, case2, SMALL_PIECES)
    assert not np.array_equal(a["tables"], b["tables"])
    assert np.array_equal(bits(a["out"]), bits(b["out"]))


def test_bf16_output_rounds_the_f32_result(pk):
    case = synth.decode_case("c3s")
    for schedule in (DEFAULT, TINY_PIECES):
        f32 = product_decode_step(pk, case, schedule)
        b16 = product_decode_step(pk, case, schedule, out_dtype=torch.bfloat16)
        assert np.array_equal(b16["out"], synth.f32_to_bf16_bits(f32["out"]))


def _edge_case(lens, b, hq=32, hkv=8, d=128, seed=31):
    lens = np.asarray(lens, dtype=np.int32)
    rng = np.random.default_rng(seed)
    nb = int(sum(-(-int(L) // b) for L in lens)) + 5
    total = int(lens.sum())
    return dict(cfg=dict(num_kv_heads=hkv, num_q_heads=hq, head_dim=d, block_size=b, dtype="bf16"),
                lengths=lens, free_order=rng.permutation(nb).astype(np.int32), num_blocks=nb,
                keys=synth.f32_to_bf16_bits(rng.standard_normal((total, hkv, d), dtype=np.float32)),
                values=synth.f32_to_bf16_bits(rng.standard_normal((total, hkv, d), dtype=np.float32)),
                q=synth.f32_to_bf16_bits(rng.standard_normal((len(lens), hq, d), dtype=np.float32)),
                offsets=np.concatenate([[0], np.cumsum(lens)]), scale=synth.default_scale(d))


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("cap,parts", [(25, 4), (7, 15), (3, 34), (1, 100)])
def test_merge_of_many_pieces(pk, dt, d, cap, parts):
    """Rows cut into 4, 15, 34 and 100 pieces: the merge launch takes a row's
    pieces in batches (4, 16 or 32 at a time for head_dim 128, 4 or 8 for
    64), so these rows cover one batch of each size and several batches of
    the largest, against the oracle."""
    lens = np.array([1600, 1599, 5, 300, 0], dtype=np.int32)
    case = _edge_case(lens, 16, hq=8, hkv=4, d=d, seed=71)
    if dt == "f32":
        rng = np.random.default_rng(72)
        total = int(lens.sum())
        case["cfg"]["dtype"] = "f32"
        case["keys"] = rng.standard_normal((total, 4, d), dtype=np.float32)
        case["values"] = rng.standard_normal((total, 4, d), dtype=np.float32)
        case["q"] = rng.standard_normal((len(lens), 8, d), dtype=np.float32)
    plan = pk.decode_plan(lens, 4, max_piece_tiles=cap, schedule=pk.SCHEDULE_LPT)
    assert int(plan.merges()[:, 2].max()) == parts
    log(f"merge of {parts} pieces {dt} D={d}")
    got = product_decode_step(pk, case, (None, cap, pk.SCHEDULE_LPT))
    ref = oracle_decode_step(case)
    assert np.array_equal(got["out"][4], np.zeros_like(got["out"][4]))
    assert_close(got["out"], ref["out"], dt, f"merge {parts} pieces {dt}")


def _f32_case(lens, b, hq, hkv, d, seed):
    """_edge_case with float32 keys, values and queries (standard normal)."""
    case = _edge_case(lens, b, hq=hq, hkv=hkv, d=d, seed=seed)
    rng = np.random.default_rng(seed + 1)
    total = int(np.asarray(lens).sum())
    case["cfg"]["dtype"] = "f32"
    case["keys"] = rng.standard_normal((total, hkv, d), dtype=np.float32)
    case["values"] = rng.standard_normal((total, hkv, d), dtype=np.float32)
    case["q"] = rng.standard_normal((len(lens), hq, d), dtype=np.float32)
    return case


@pytest.mark.parametrize("b,d,hq,hkv", [(16, 128, 32, 8), (32, 128, 64, 4), (8, 64, 6, 3), (2, 128, 8, 8),
                                        (4, 64, 20, 2), (1, 128, 16, 4)])
def test_f32_decode_matches_oracle(pk, b, d, hq, hkv):
    """The fp32 path (both contractions on fp32 MFMA) against the float64
    oracle at fp32's tolerance: groups of 1 to 16 query heads per KV head, a
    KV-head count that leaves wavefronts idle, head_dim 64 and 128, every
    block size, contexts that are empty, one token, tile and block multiples
    and one past them, whole and cut into pieces, the append separate and
    fused."""
    lens = [0, 1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 0, 255, 256, 257, 1023, 1025]
    case = _f32_case(lens, b, hq, hkv, d, seed=90 + b)
    ref = oracle_decode_step(case)
    for schedule in (DEFAULT, TINY_PIECES, SMALL_PIECES):
        for fused in (False, True):
            log(f"f32 B={b} D={d} {hq}/{hkv} schedule={schedule} fused={fused}")
            got = product_decode_step(pk, case, schedule, fused=fused)
            for s in np.flatnonzero(np.asarray(lens) == 0):
                assert np.array_equal(got["out"][s], np.zeros((hq, d), np.float32))
            stats = assert_close(got["out"], ref["out"], "f32", f"f32 B={b} D={d} {schedule} fused={fused}")
            log(f"  max|err|={stats['max_abs']:.3g}")


@pytest.mark.parametrize("b", [8, 16])
@pytest.mark.parametrize("kind", ["lpt", "chunks"])
def test_advanced_plan_matches_oracle(pk, b, kind):
    """A plan built once and carried forward by pa_decode_plan_advance over
    four steps of lengths growing by one (crossing tile and block boundaries
    on the way) decodes like the oracle at every step."""
    base = np.array([1, 15, 16, 17, 31, 32, 33, 100, 255, 256, 257, 700, 0, 2, 47], dtype=np.int32)
    steps = 4
    full = np.where(base > 0, base + steps, 0).astype(np.int32)
    case = _edge_case(full, b, seed=91)
    got = product_decode_step(pk, case)
    ref = oracle_decode_step(case)
    assert np.array_equal(got["tables"], ref["tables"])
    sched = pk.SCHEDULE_LPT if kind == "lpt" else pk.SCHEDULE_CHUNKS
    plan = pk.decode_plan(base, 8, 16, 3, schedule=sched, block_size=b)
    hq, d = case["cfg"]["num_q_heads"], case["cfg"]["head_dim"]
    ws = torch.full((max(pk.decode_workspace_bytes(plan, hq, d), 256) // 4,), float("nan"), device="cuda")
    for k in range(steps + 1):
        lens = np.where(base > 0, base + k, 0).astype(np.int32)
        if k:
            assert plan.advance(lens)
        plan.check_lens(lens)
        log(f"advanced plan {kind} B={b} step {k}: {plan.num_jobs} jobs, {plan.info.num_tiles} tiles")
        out = torch.full((len(base), hq, d), float("nan"), device="cuda")
        pk.decode(got["pool"], got["q_dev"], to_dev(got["tables"]), to_dev(lens), case["scale"], plan,
                  plan.to_device(), ws, out=out)
        torch.cuda.synchronize()
        expect = oracle.decode_attention(case["q"], ref["kpool"], ref["vpool"], ref["tables"], lens, case["scale"])
        assert_close(to_host(out), expect, "bf16", f"advanced plan {kind} B={b} step {k}")


@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32])
def test_edge_lengths(pk, b):
    """Empty contexts, one token, exact block/tile multiples and one past
    them, pieces of 64 tiles (8 * B below B = 8), and a context filling its
    table exactly."""
    lens = [0, 1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 0, 255, 256, 257, 1023, 1024, 1025, 2100]
    case = _edge_case(lens, b)
    ref = oracle_decode_step(case)
    for schedule in (DEFAULT, FEW_WG, TINY_PIECES, (5, 64)):
        log(f"edge lengths B={b} schedule={schedule}")
        got = product_decode_step(pk, case, schedule)
        for s in np.flatnonzero(np.asarray(lens) == 0):
            assert np.array_equal(got["out"][s], np.zeros((32, 128), np.float32))
        assert_close(got["out"], ref["out"], "bf16", f"edge/B{b}/{schedule}")


@pytest.mark.parametrize("hq,hkv", [(6, 3), (16, 16), (20, 2), (5, 5)])
def test_head_layouts(pk, hq, hkv):
    """KV-head counts that do not fill a block of four, MHA with 16 heads,
    and a group of 10 query heads per KV head."""
    case = _edge_case([5, 40, 130, 17], 16, hq=hq, hkv=hkv)
    ref = oracle_decode_step(case)
    for schedule in (DEFAULT, TINY_PIECES):
        got = product_decode_step(pk, case, schedule)
        assert_close(got["out"], ref["out"], "bf16", f"heads {hq}/{hkv} {schedule}")


def test_single_token_context_returns_value_exactly(pk):
    """L = 1: softmax weight 1, so the output is the appended value row."""
    case = dict(synth.decode_case("c1"))
    case["lengths"] = np.ones(4, dtype=np.int32)
    case["offsets"] = np.arange(5)
    got = product_decode_step(pk, case, DEFAULT)
    g = case["cfg"]["num_q_heads"] // case["cfg"]["num_kv_heads"]
    for s in range(4):
        for h in range(case["cfg"]["num_q_heads"]):
            assert np.array_equal(got["out"][s, h], case["values"][s, h // g])


# ------------------------------------------------------- prefix sharing, CoW
@pytest.mark.parametrize("b", [1, 4, 8, 16, 32])
def test_prefix_sharing_matches_oracle_and_private_copies(pk, b):
    log(f"prefix sharing c5s B={b}")
    case = synth.prefix_case("c5s", b)
    got = product_prefix(pk, case, SMALL_PIECES)
    ref = oracle_prefix(case)
    assert np.array_equal(got["tables"], ref["tables"])
    assert np.array_equal(got["cows"].reshape(-1, 2), ref["cows"])
    pre = case["cfg"]["prefix_len"]
    n = case["cfg"]["samples"]
    expect_cows = 0 if pre % b == 0 else case["cfg"]["num_prompts"] * (n - 1)
    assert len(ref["cows"]) == expect_cows
    assert np.array_equal(bits(to_host(got["kpool"])), bits(ref["kpool"]))
    assert np.array_equal(bits(to_host(got["vpool"])), bits(ref["vpool"]))
    assert_close(got["out"], ref["out"], "bf16", f"c5s/B{b}")
    private = product_prefix(pk, case, SMALL_PIECES, shared=False)
    assert np.array_equal(bits(got["out"]), bits(private["out"]))


@pytest.mark.parametrize("b", [8, 16, 32])
def test_shared_kv_cache_policy_gives_identical_output(pk, b):
    """PA_DECODE_SHARED_KV only changes how K/V loads use the caches."""
    case = synth.prefix_case("c5s", b)
    got = product_prefix(pk, case, SMALL_PIECES)
    assert got["stats"]["shared_blocks"] > 0
    args = (pk, got["pool"], to_dev(case["q"]), got["tables"], got["lens"], case["scale"], SMALL_PIECES)
    streamed = to_host(gpu_decode(*args, shared_kv=False))
    cached = to_host(gpu_decode(*args, shared_kv=True))
    assert np.array_equal(bits(streamed), bits(cached))
    assert np.array_equal(bits(streamed), bits(got["out"]))


@pytest.mark.parametrize("b", [2, 4, 8, 16, 32])
@pytest.mark.parametrize("schedule", [DEFAULT, SMALL_PIECES, TINY_PIECES])
def test_cascade_decode_matches_oracle(pk, b, schedule):
    """Shared prefixes read once per group of samples (pa_decode_plan_prefix):
    same outputs as the oracle within tolerance, and as the per-sequence plan
    within the accumulation-order difference."""
    log(f"cascade c5s B={b} schedule={schedule}")
    case = synth.prefix_case("c5s", b)
    got = product_prefix(pk, case, schedule, cascade=True)
    assert got["plan"].num_groups > 0
    ref = oracle_prefix(case)
    stats = assert_close(got["out"], ref["out"], "bf16", f"cascade c5s/B{b}/{schedule}")
    log(f"  max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g} groups={got['plan'].num_groups}")
    plain = product_prefix(pk, case, schedule)
    assert np.abs(got["out"] - plain["out"]).max() < 2e-3


@pytest.mark.parametrize("b", [8, 16, 32])
@pytest.mark.parametrize("schedule", [(512, 0), (64, 0), (72, 0), (64, 3), (7, 3)])
def test_wide_prefix_cascade_matches_oracle(pk, b, schedule):
    """Prompts sampled 14 times: each prefix is shared by four groups (three of
    four samples and one of two), which the plan places on one die of the grid
    when the grid is a multiple of 8 of at least 64 workgroups (512, 64, 72),
    reading each prefix once per KV head for the set of four groups (wide
    jobs: the workgroup's wavefronts exchange tiles through LDS), and by the
    chunk schedule otherwise (7).  Same outputs as the oracle within
    tolerance and as the per-sequence plan within the accumulation-order
    difference."""
    log(f"cascade c5w B={b} schedule={schedule}")
    case = synth.prefix_case("c5w", b)
    got = product_prefix(pk, case, schedule, cascade=True)
    assert got["plan"].num_groups > 0 and got["plan"].info.flags == pk.PA_DECODE_SHARED_KV
    if schedule == (512, 0):
        assert got["plan"].info.wide_jobs > 0
    ref = oracle_prefix(case)
    stats = assert_close(got["out"], ref["out"], "bf16", f"cascade c5w/B{b}/{schedule}")
    log(f"  max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g} groups={got['plan'].num_groups} "
        f"wide jobs={got['plan'].info.wide_jobs}")
    plain = product_prefix(pk, case, schedule)
    assert np.abs(got["out"] - plain["out"]).max() < 2e-3


@pytest.mark.parametrize("b", [8, 16, 32])
def test_cascade_decode_with_first_tile_entries(pk, b):
    log(f"cascade c5s B={b} with first-tile entries")
    case = synth.prefix_case("c5s", b)
    got = product_prefix(pk, case, SMALL_PIECES, cascade=True)
    seqs = np.arange(len(got["lens"]))
    out, plan = cascade_decode(pk, got["pool"], to_dev(case["q"]), got["tables"], got["lens"], case["scale"],
                               got["bm"], seqs, SMALL_PIECES, first_blocks=True)
    assert plan.info.flags & pk.PA_DECODE_FIRST_BLOCKS
    assert np.array_equal(bits(to_host(out)), bits(got["out"]))


@pytest.mark.parametrize("name,schedule", [("c5s", SMALL_PIECES), ("c5w", (512, 0))])
def test_cascade_decode_with_fused_append(pk, name, schedule):
    """The append fused into a shared-prefix decode: the appended tokens sit in
    each sample's own tiles; pools byte-identical to the separate write.  c5w
    on the full grid reads its prefixes with wide jobs."""
    log(f"cascade {name} fused append, schedule={schedule}")
    case = synth.prefix_case(name, 16)
    got = product_prefix(pk, case, schedule)
    bm, pool, lens = got["bm"], got["pool"], got["lens"]
    nseq = len(lens)
    # one more token per sample: block manager slots, then fused vs separate
    rng = np.random.default_rng(7)
    hkv, d = case["cfg"]["num_kv_heads"], case["cfg"]["head_dim"]
    nk = synth.f32_to_bf16_bits(rng.standard_normal((nseq, hkv, d), dtype=np.float32))
    nv = synth.f32_to_bf16_bits(rng.standard_normal((nseq, hkv, d), dtype=np.float32))
    slots, cows = bm.append_step(np.arange(nseq))
    assert len(cows) == 0
    tables, lens2 = bm.export(np.arange(nseq), int(max(-(-int(L) // 16) for L in lens + 1)))
    k_sep, v_sep = pool.k.clone(), pool.v.clone()
    sep = pk.KvPool(k_sep, v_sep)
    pk.reshape_and_cache(sep, to_dev(nk), to_dev(nv), to_dev(np.asarray(slots, np.int64)))
    out_sep, plan = cascade_decode(pk, sep, to_dev(case["q"]), tables, lens2, case["scale"], bm, np.arange(nseq),
                                   schedule)
    assert name != "c5w" or plan.info.wide_jobs > 0
    out_fused, _ = cascade_decode(pk, pool, to_dev(case["q"]), tables, lens2, case["scale"], bm, np.arange(nseq),
                                  schedule, new_key=to_dev(nk), new_value=to_dev(nv))
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(pool.k)), bits(to_host(k_sep)))
    assert np.array_equal(bits(to_host(pool.v)), bits(to_host(v_sep)))
    assert np.array_equal(bits(to_host(out_fused)), bits(to_host(out_sep)))


def test_use_after_free_poisoning_leaves_sharers_unchanged(pk):
    """Retire one sample, overwrite every block that went back to the free
    list with NaN; the surviving samples' outputs must not change."""
    case = synth.prefix_case("c5s", 16)
    got = product_prefix(pk, case, SMALL_PIECES)
    before = got["out"].copy()
    bm = got["bm"]
    victim = 1
    others = [s for s in range(len(got["tables"])) if s != victim]
    victim_blocks = bm.table(victim).tolist()
    bm.free(victim)
    bm.check()
    freed = [b for b in victim_blocks if bm.refcount(b) == 0]
    kept = [b for b in victim_blocks if bm.refcount(b) > 0]
    assert freed and kept, "the victim owned private blocks and shared prefix blocks"
    pool = got["pool"]
    pool.k[freed] = float("nan")
    pool.v[freed] = float("nan")
    out = to_host(gpu_decode(pk, pool, to_dev(case["q"]), got["tables"], got["lens"], case["scale"], SMALL_PIECES))
    assert np.array_equal(bits(out[others]), bits(before[others]))


@pytest.mark.parametrize("name", ["c1", "c3s"])
@pytest.mark.parametrize("schedule", [DEFAULT, TINY_PIECES, FEW_WG])
def test_plan_for_other_lengths_gives_nan_not_numbers(pk, name, schedule):
    """A plan built for other context lengths than the device's (every odd
    sequence one token shorter, as a plan kept from the previous step would
    be, and one non-empty sequence planned as empty) passes the host checks,
    which cannot see device lengths.  Every job compares its sequence's
    device length with the planned one: each output element of a sequence
    whose lengths differ is NaN, whether the job writes it directly or
    through merged records, and every other sequence matches the oracle."""
    log(f"stale plan {name} schedule={schedule}")
    case = synth.decode_case(name)
    cfg = case["cfg"]
    got = product_decode_step(pk, case, schedule)
    ref = oracle_decode_step(case)
    lens = got["lens"]
    stale = lens.copy()
    stale[1::2] = np.maximum(stale[1::2] - 1, 0)
    live = np.flatnonzero(lens > 0)
    stale[live[-1]] = 0
    differ = stale != lens
    assert differ.any() and (~differ).any()
    plan, plan_dev, ws = plan_and_workspace(pk, stale, cfg["num_kv_heads"], cfg["num_q_heads"], cfg["head_dim"],
                                            *schedule)
    for fused in (False, True):
        out = torch.zeros(tuple(got["q_dev"].shape), dtype=torch.float32, device="cuda")
        nk = nv = None
        if fused:
            # The appended rows are already in the pool; storing them again
            # from the device lengths leaves it unchanged.
            last = np.array([case["offsets"][s + 1] - 1 if lens[s] > 0 else 0 for s in range(len(lens))])
            nk, nv = to_dev(case["keys"][last]), to_dev(case["values"][last])
        pk.decode(got["pool"], got["q_dev"], to_dev(got["tables"]), to_dev(lens), case["scale"], plan, plan_dev, ws,
                  out=out, new_key=nk, new_value=nv)
        o = to_host(out)
        assert np.all(np.isnan(o[differ])), f"fused={fused}: a sequence planned for another length is not all NaN"
        assert_close(o[~differ], ref["out"][~differ], cfg["dtype"], f"stale plan {name}/{schedule}/fused={fused}")
        torch.cuda.synchronize()
        assert np.array_equal(bits(to_host(got["pool"].k)), bits(ref["kpool"]))
        assert np.array_equal(bits(to_host(got["pool"].v)), bits(ref["vpool"]))


def _at_block_size(case: dict, b: int) -> dict:
    """The same lengths and K/V with pools of block size b (a seeded pool of
    the same slack and a shuffled free list)."""
    out = dict(case)
    out["cfg"] = dict(case["cfg"], block_size=b)
    nb = synth.pool_blocks_for(case["lengths"], b)
    out["num_blocks"] = nb
    out["free_order"] = np.random.default_rng(500 + b).permutation(nb).astype(np.int32)
    return out


@pytest.mark.parametrize("b", [1, 2, 4])
@pytest.mark.parametrize("schedule", [DEFAULT, FEW_WG, SMALL_PIECES])
def test_small_block_sizes_match_oracle(pk, b, schedule):
    """Blocks of 1, 2 and 4 slots (a 16-token tile spans 16, 8 or 4 blocks;
    the pages' block-size sweep starts at 1): the batch-256-shaped GQA case
    (c3s, 24 sequences) through the block manager, the cache kernels and the
    decode launch, separate and fused append; tables, slots and pools
    bit-exact, outputs within tolerance of the oracle; fp32 too (c1)."""
    for name in ("c3s", "c1"):
        log(f"block size {b} {name} schedule={schedule}")
        case = _at_block_size(synth.decode_case(name), b)
        ref = oracle_decode_step(case)
        for fused in (False, True):
            got = product_decode_step(pk, case, schedule, fused=fused)
            assert np.array_equal(got["tables"], ref["tables"])
            assert got["new_slots"] == ref["new_slots"]
            assert np.array_equal(bits(got["kpool"]), bits(ref["kpool"]))
            assert np.array_equal(bits(got["vpool"]), bits(ref["vpool"]))
            stats = assert_close(got["out"], ref["out"], case["cfg"]["dtype"], f"B={b} {name} {schedule} fused={fused}")
            log(f"  fused={fused} max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g}")


@pytest.mark.parametrize("b", [1, 2, 4])
def test_small_block_sizes_refuse_jobs_past_the_table_window(pk, b):
    """Below 8 slots per block a job may cover at most 8 * B tiles; a plan
    with longer jobs is refused before any launch."""
    case = _at_block_size(synth.decode_case("c3s"), b)
    got = product_decode_step(pk, case, DEFAULT)
    cfg = case["cfg"]
    plan = pk.decode_plan(got["lens"], cfg["num_kv_heads"], num_workgroups=4, max_piece_tiles=64,
                          schedule=pk.SCHEDULE_LPT)
    assert plan.info.max_job_tiles > 8 * b
    nbytes = max(pk.decode_workspace_bytes(plan, cfg["num_q_heads"], cfg["head_dim"]), 256)
    ws = torch.empty(nbytes // 4, device="cuda")
    with pytest.raises(pk.PaError, match="at most"):
        pk.decode(got["pool"], got["q_dev"], to_dev(got["tables"]), to_dev(got["lens"]), case["scale"], plan,
                  plan.to_device(), ws)
