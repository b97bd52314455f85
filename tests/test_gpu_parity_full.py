"""GPU parity at full size, in the launch configuration bench.py times.

Each workload runs at its full size with the device-default schedule
(resident workgroups, automatic piece length), through the C++ block manager,
pa_copy_blocks / pa_reshape_and_cache and pa_decode, and the decode step once
more as bench.py times it (the append fused into pa_decode, first-tile
entries in the plan).  Block tables, slots and
both pools are compared in full: bit-exact.  Attention outputs are compared
with the float64 oracle element by element for every sequence of the batch
(the oracle runs one sequence at a time, a few seconds per workload); the
tolerances are those of every parity test (bf16 max |err| <= 1e-2, mean
<= 1e-3).  Each test also logs the sequences the plan cuts into the most
pieces and their own errors, the cases a schedule bug would hit first."""
import numpy as np
import pytest
import torch

import synth
from flows import (assert_close, bits, oracle_decode_step, oracle_prefix, product_decode_step, product_prefix)

pytestmark = pytest.mark.gpu

DEFAULT = (None, 0)


@pytest.fixture(scope="module")
def pk():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import paged_kv_cache_115_amd as m
    return m


def log(msg):
    print(msg, flush=True)


def most_cut(pk, lens: np.ndarray, hkv: int, n: int = 2) -> list:
    """The n sequences the default plan cuts into the most pieces."""
    plan = pk.decode_plan(np.asarray(lens), hkv)
    merges = plan.merges()
    cut = merges[merges[:, 2] > 1]
    seen = []
    for s in cut[np.argsort(-cut[:, 2], kind="stable"), 0].tolist():
        if s not in seen:
            seen.append(int(s))
    return seen[:n]


def compare_all(got: np.ndarray, ref: np.ndarray, dt: str, where: str, watch: list) -> None:
    """Every output against the oracle; the watched sequences are also logged alone."""
    assert got.shape == ref.shape
    stats = assert_close(got, ref, dt, where)
    log(f"  {where}: all {got.shape[0]} sequences max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g}")
    for s in watch:
        e = np.abs(got[s].astype(np.float64) - ref[s])
        log(f"    seq {s}: max|err|={e.max():.3g}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_full_size_decode_step(pk, name):
    case = synth.decode_case(name)
    cfg = case["cfg"]
    watch = most_cut(pk, case["lengths"], cfg["num_kv_heads"])
    log(f"full-size decode {name}: {len(case['lengths'])} seqs, {int(case['lengths'].sum())} tokens")
    got = product_decode_step(pk, case, DEFAULT)
    ref = oracle_decode_step(case)
    assert np.array_equal(got["tables"], ref["tables"])
    assert got["new_slots"] == ref["new_slots"]
    assert all(np.array_equal(a, b) for a, b in zip(got["pre_slots"], ref["pre_slots"]))
    assert np.array_equal(bits(got["kpool"]), bits(ref["kpool"]))
    assert np.array_equal(bits(got["vpool"]), bits(ref["vpool"]))
    compare_all(got["out"], ref["out"], cfg["dtype"], name, watch)
    # The step bench.py times: the append fused into pa_decode, with the
    # plan's first-tile entries.  Pools as the oracle's, output bitwise that
    # of the three calls.
    log(f"full-size decode {name}: append fused, first-tile entries")
    fused = product_decode_step(pk, case, DEFAULT, fused=True, first_blocks=True)
    assert np.array_equal(bits(fused["kpool"]), bits(ref["kpool"]))
    assert np.array_equal(bits(fused["vpool"]), bits(ref["vpool"]))
    assert np.array_equal(bits(fused["out"]), bits(got["out"]))
    compare_all(fused["out"], ref["out"], cfg["dtype"], f"{name} fused", watch)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("b", [8, 16, 32])
def test_full_size_prefix_sharing(pk, b):
    case = synth.prefix_case("c5", b)
    hkv = case["cfg"]["num_kv_heads"]
    lens = (case["cfg"]["prefix_len"] + case["tail_lengths"]).astype(np.int32)
    watch = most_cut(pk, lens, hkv)
    log(f"full-size prefix sharing B={b}: {len(lens)} seqs")
    got = product_prefix(pk, case, DEFAULT)
    ref = oracle_prefix(case)
    assert np.array_equal(got["tables"], ref["tables"])
    assert np.array_equal(got["cows"].reshape(-1, 2), ref["cows"].reshape(-1, 2))
    expected_copies = case["cfg"]["num_prompts"] * (case["cfg"]["samples"] - 1) if case["cfg"]["prefix_len"] % b else 0
    assert len(ref["cows"]) == expected_copies
    from flows import to_host
    assert np.array_equal(bits(to_host(got["kpool"])), bits(ref["kpool"]))
    assert np.array_equal(bits(to_host(got["vpool"])), bits(ref["vpool"]))
    compare_all(got["out"], ref["out"], "bf16", f"c5 B={b}", watch)
    # The same batch with each shared prefix read once per group of samples.
    from flows import cascade_decode, to_dev
    out, plan = cascade_decode(pk, got["pool"], to_dev(case["q"]), got["tables"], got["lens"], case["scale"],
                               got["bm"], np.arange(len(lens)))
    assert plan.num_groups == case["cfg"]["num_prompts"] * -(-hkv // 4)
    compare_all(to_host(out), ref["out"], "bf16", f"c5 B={b} cascade", watch)


def test_full_size_prefix_cache_requests(pk):
    """c6 at full size: 256 requests over four 2,000-token system prompts,
    admitted through the library's prefix cache and the oracle's model side by
    side (slots, reuse and tables equal; only non-reused rows written; both
    pools bit-exact), then decoded with the cascade plan that bench.py times
    and with per-request plans; every request against the oracle."""
    import oracle
    from flows import cascade_decode, gpu_decode, to_dev, to_host
    case = synth.prefix_cache_case("c6")
    cfg = case["cfg"]
    b, hkv, d, dt = cfg["block_size"], cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    prompts = case["prompts"]
    S = len(prompts)
    nb = sum(-(-(len(p) + 1) // b) for p in prompts)
    order = np.random.default_rng(cfg["seed"]).permutation(nb).astype(np.int32)
    log(f"c6 full size: {S} requests, {nb} blocks")
    om = oracle.BlockManagerModel(nb, b, order)
    om.enable_prefix_cache()
    bm = pk.BlockManager(nb, b, order)
    bm.enable_prefix_cache()
    ok, ov = synth.nan_fill((nb, b, hkv, d), dt), synth.nan_fill((nb, b, hkv, d), dt)
    kd, vd = to_dev(ok), to_dev(ov)
    pool = pk.KvPool(kd, vd)
    for r, p in enumerate(prompts):
        ms, mc = om.append_prompt(r, p)
        ps, pc = bm.append_prompt(r, p)
        assert pc == mc and ps.tolist() == ms, r
        rk, rv = synth.token_rows(p, hkv, d, dt, start=mc)
        oracle.reshape_and_cache(ok, ov, rk, rv, np.array(ms[mc:], dtype=np.int64))
        pk.reshape_and_cache(pool, to_dev(rk), to_dev(rv), to_dev(ps[mc:]))
    st = bm.stats()
    assert st["prefix_hit_tokens"] == om.stats()["prefix_hit_tokens"] > 0
    bm.check()
    seqs = np.arange(S)
    maxb = max(len(bm.table(s)) for s in seqs)
    tables, lens = bm.export(seqs, maxb)
    for s in seqs:
        assert tables[s, :len(om.table(s))].tolist() == om.table(s)
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(kd)), bits(ok)) and np.array_equal(bits(to_host(vd)), bits(ov))
    watch = most_cut(pk, lens, hkv)
    ref = oracle.decode_attention(case["q"], ok, ov, tables, lens, case["scale"])
    out, plan = cascade_decode(pk, pool, to_dev(case["q"]), tables, lens, case["scale"], bm, seqs)
    assert plan.num_groups > 0
    compare_all(to_host(out), ref, dt, "c6 cascade", watch)
    out2 = to_host(gpu_decode(pk, pool, to_dev(case["q"]), tables, lens, case["scale"], shared_kv=True))
    compare_all(out2, ref, dt, "c6 per-request plans", watch)
