"""GPU parity: the HIP path against the float64 oracle on identical seeded
inputs.  Cache kernels bit-exact; attention within the stated tolerances;
invariances bitwise."""
import numpy as np
import pytest
import torch

import oracle
import synth

from flows import (assert_close, bits, gpu_decode, oracle_decode_step, oracle_prefix, product_decode_step,
                   product_prefix, to_dev, to_host)

pytestmark = pytest.mark.gpu


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
                                        ("bf16", 32, 2, 128), ("f32", 32, 3, 128)])
def test_reshape_and_cache_bit_exact(pk, dt, b, hkv, d):
    log(f"reshape_and_cache dt={dt} B={b} Hkv={hkv} D={d}")
    rng = np.random.default_rng(21)
    nb = 61
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


@pytest.mark.parametrize("dt,b,hkv,d", [("bf16", 16, 8, 128), ("bf16", 32, 8, 128), ("f32", 8, 4, 64)])
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
DECODE_CASES = [("c1", 0), ("c1", 16), ("c1", 32), ("c2s", 0), ("c2s", 64), ("c3s", 256), ("c3s", 64),
                ("c3s", 0), ("c4s", 512), ("c4s", 128)]


@pytest.mark.parametrize("name,partition", DECODE_CASES)
def test_decode_step_matches_oracle(pk, name, partition):
    log(f"decode step {name} partition={partition}")
    case = synth.decode_case(name)
    dt = case["cfg"]["dtype"]
    got = product_decode_step(pk, case, partition)
    ref = oracle_decode_step(case)
    assert np.array_equal(got["tables"], ref["tables"])
    assert [list(x) for x in got["pre_slots"]] == [list(x) for x in ref["pre_slots"]]
    assert got["new_slots"] == ref["new_slots"]
    assert np.array_equal(bits(got["kpool"]), bits(ref["kpool"]))
    assert np.array_equal(bits(got["vpool"]), bits(ref["vpool"]))
    stats = assert_close(got["out"], ref["out"], dt, f"{name}/P{partition}")
    log(f"  max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g}")


def test_decode_is_deterministic_and_partition_independent_within_tolerance(pk):
    case = synth.decode_case("c3s")
    a = product_decode_step(pk, case, 64)
    again = gpu_decode(pk, a["pool"], a["q_dev"], a["tables"], a["lens"], case["scale"], 64)
    assert np.array_equal(to_host(again), a["out"])
    b = product_decode_step(pk, case, 0)
    assert np.abs(a["out"] - b["out"]).max() < 2e-3


def test_physical_block_permutation_is_bitwise_invariant(pk):
    """Same logical content through two different free-list orders."""
    case = synth.decode_case("c3s")
    a = product_decode_step(pk, case, 128)
    case2 = dict(case)
    case2["free_order"] = np.random.default_rng(99).permutation(case["num_blocks"]).astype(np.int32)
    b = product_decode_step(pk, case2, 128)
    assert not np.array_equal(a["tables"], b["tables"])
    assert np.array_equal(bits(a["out"]), bits(b["out"]))


def test_bf16_output_rounds_the_f32_result(pk):
    case = synth.decode_case("c3s")
    f32 = product_decode_step(pk, case, 64)
    b16 = product_decode_step(pk, case, 64, out_dtype=torch.bfloat16)
    expect = synth.f32_to_bf16_bits(f32["out"])
    assert np.array_equal(b16["out"], expect)


def test_edge_lengths(pk):
    """Empty context, one token, exact block/tile/partition multiples, one
    past them, and a context filling its table exactly."""
    lens = np.array([0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513], dtype=np.int32)
    hq, hkv, d, b = 32, 8, 128, 16
    rng = np.random.default_rng(31)
    nb = int(sum(-(-int(L) // b) for L in lens)) + 5
    order = rng.permutation(nb).astype(np.int32)
    total = int(lens.sum())
    case = dict(cfg=dict(num_kv_heads=hkv, num_q_heads=hq, head_dim=d, block_size=b, dtype="bf16"),
                lengths=lens, free_order=order, num_blocks=nb,
                keys=synth.f32_to_bf16_bits(rng.standard_normal((total, hkv, d), dtype=np.float32)),
                values=synth.f32_to_bf16_bits(rng.standard_normal((total, hkv, d), dtype=np.float32)),
                q=synth.f32_to_bf16_bits(rng.standard_normal((len(lens), hq, d), dtype=np.float32)),
                offsets=np.concatenate([[0], np.cumsum(lens)]), scale=synth.default_scale(d))
    ref = oracle_decode_step(case)
    for partition in (0, 16, 32, 256):
        log(f"edge lengths partition={partition}")
        got = product_decode_step(pk, case, partition)
        assert np.array_equal(got["out"][0], np.zeros((hq, d), np.float32))
        assert_close(got["out"], ref["out"], "bf16", f"edge/P{partition}")


def test_single_token_context_returns_value_exactly(pk):
    """L = 1: softmax weight 1, so the output is the appended value row."""
    case = synth.decode_case("c1")
    case = dict(case)
    case["lengths"] = np.ones(4, dtype=np.int32)
    case["offsets"] = np.arange(5)
    got = product_decode_step(pk, case, 0)
    g = case["cfg"]["num_q_heads"] // case["cfg"]["num_kv_heads"]
    for s in range(4):
        for h in range(case["cfg"]["num_q_heads"]):
            assert np.array_equal(got["out"][s, h], case["values"][s, h // g])


# ------------------------------------------------------- prefix sharing, CoW
@pytest.mark.parametrize("b", [8, 16, 32])
def test_prefix_sharing_matches_oracle_and_private_copies(pk, b):
    log(f"prefix sharing c5s B={b}")
    case = synth.prefix_case("c5s", b)
    got = product_prefix(pk, case, 64)
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
    private = product_prefix(pk, case, 64, shared=False,
                             private_order=None)
    assert np.array_equal(bits(got["out"]), bits(private["out"]))


def test_use_after_free_poisoning_leaves_sharers_unchanged(pk):
    """Retire one sample, overwrite every block that went back to the free
    list with NaN; the surviving samples' outputs must not change."""
    case = synth.prefix_case("c5s", 16)
    got = product_prefix(pk, case, 64)
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
    out = gpu_decode(pk, pool, to_dev(case["q"]), got["tables"], got["lens"], case["scale"], 64)
    out = to_host(out)
    assert np.array_equal(bits(out[others]), bits(before[others]))
