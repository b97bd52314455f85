"""GPU parity at full size, in the launch configuration bench.py times.

Each workload runs at its full size with the device-default schedule
(resident workgroups, automatic piece length), through the C++ block manager,
pa_copy_blocks / pa_reshape_and_cache and pa_decode, and the decode step once
more as bench.py times it (the append fused into pa_decode, first-tile
entries in the plan).  Block tables, slots and
both pools are compared in full: bit-exact.  Attention outputs are compared on
sampled sequences that the float64 oracle computes one by one: the longest,
the shortest, the ones the plan cuts into the most pieces, and a seeded random
few; tolerances as everywhere (bf16 max |err| <= 1e-2, mean <= 1e-3)."""
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


def sample_seqs(pk, lens: np.ndarray, hkv: int, seed: int, n_random: int = 4) -> list:
    lens = np.asarray(lens)
    live = np.flatnonzero(lens > 0)
    plan = pk.decode_plan(lens, hkv)
    merges = plan.merges()
    cut = merges[merges[:, 2] > 1]
    most_cut = [int(s) for s in cut[np.argsort(-cut[:, 2], kind="stable"), 0]][:2]
    rng = np.random.default_rng(seed)
    picks = [int(live[np.argmax(lens[live])]), int(live[np.argmin(lens[live])])] + most_cut
    picks += [int(s) for s in rng.choice(live, size=min(n_random, live.size), replace=False)]
    return sorted(set(picks))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_full_size_decode_step(pk, name):
    case = synth.decode_case(name)
    cfg = case["cfg"]
    seqs = sample_seqs(pk, case["lengths"], cfg["num_kv_heads"], seed=7)
    log(f"full-size decode {name}: {len(case['lengths'])} seqs, {int(case['lengths'].sum())} tokens, "
        f"sampled {seqs}")
    got = product_decode_step(pk, case, DEFAULT)
    ref = oracle_decode_step(case, seqs=seqs)
    assert np.array_equal(got["tables"], ref["tables"])
    assert got["new_slots"] == ref["new_slots"]
    assert all(np.array_equal(a, b) for a, b in zip(got["pre_slots"], ref["pre_slots"]))
    assert np.array_equal(bits(got["kpool"]), bits(ref["kpool"]))
    assert np.array_equal(bits(got["vpool"]), bits(ref["vpool"]))
    assert np.all(np.isfinite(got["out"]))
    stats = assert_close(got["out"][seqs], ref["out"][seqs], cfg["dtype"], name)
    log(f"  max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g}")
    # The step bench.py times: the append fused into pa_decode, with the
    # plan's first-tile entries.  Pools as the oracle's, output bitwise that
    # of the three calls.
    log(f"full-size decode {name}: append fused, first-tile entries")
    fused = product_decode_step(pk, case, DEFAULT, fused=True, first_blocks=True)
    assert np.array_equal(bits(fused["kpool"]), bits(ref["kpool"]))
    assert np.array_equal(bits(fused["vpool"]), bits(ref["vpool"]))
    assert np.array_equal(bits(fused["out"]), bits(got["out"]))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("b", [8, 16, 32])
def test_full_size_prefix_sharing(pk, b):
    case = synth.prefix_case("c5", b)
    hkv = case["cfg"]["num_kv_heads"]
    lens = (case["cfg"]["prefix_len"] + case["tail_lengths"]).astype(np.int32)
    seqs = sample_seqs(pk, lens, hkv, seed=8)
    log(f"full-size prefix sharing B={b}: {len(lens)} seqs, sampled {seqs}")
    got = product_prefix(pk, case, DEFAULT)
    ref = oracle_prefix(case, seqs=seqs)
    assert np.array_equal(got["tables"], ref["tables"])
    assert np.array_equal(got["cows"].reshape(-1, 2), ref["cows"].reshape(-1, 2))
    expected_copies = case["cfg"]["num_prompts"] * (case["cfg"]["samples"] - 1) if case["cfg"]["prefix_len"] % b else 0
    assert len(ref["cows"]) == expected_copies
    from flows import to_host
    assert np.array_equal(bits(to_host(got["kpool"])), bits(ref["kpool"]))
    assert np.array_equal(bits(to_host(got["vpool"])), bits(ref["vpool"]))
    assert np.all(np.isfinite(got["out"]))
    stats = assert_close(got["out"][seqs], ref["out"][seqs], "bf16", f"c5 B={b}")
    log(f"  max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g}")
    # The same batch with each shared prefix read once per group of samples.
    from flows import cascade_decode, to_dev
    out, plan = cascade_decode(pk, got["pool"], to_dev(case["q"]), got["tables"], got["lens"], case["scale"],
                               got["bm"], np.arange(len(lens)))
    assert plan.num_groups == case["cfg"]["num_prompts"] * -(-hkv // 4)
    out = to_host(out)
    assert np.all(np.isfinite(out))
    stats = assert_close(out[seqs], ref["out"][seqs], "bf16", f"c5 B={b} cascade")
    log(f"  cascade max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g}")


def test_full_size_prefix_cache_requests(pk):
    """c6 at full size: 256 requests over four 2,000-token system prompts,
    admitted through the library's prefix cache and the oracle's model side by
    side (slots, reuse and tables equal; only non-reused rows written; both
    pools bit-exact), then decoded with the cascade plan that bench.py times
    and with per-request plans; sampled requests against the oracle."""
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
    sample = sample_seqs(pk, lens, hkv, 6)
    ref = oracle.decode_attention(case["q"], ok, ov, tables, lens, case["scale"], seqs=sample)
    out, plan = cascade_decode(pk, pool, to_dev(case["q"]), tables, lens, case["scale"], bm, seqs)
    assert plan.num_groups > 0
    out = to_host(out)
    assert np.all(np.isfinite(out))
    stats = assert_close(out[sample], ref[sample], dt, "c6 cascade")
    log(f"  cascade max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g}")
    out2 = to_host(gpu_decode(pk, pool, to_dev(case["q"]), tables, lens, case["scale"], shared_kv=True))
    stats = assert_close(out2[sample], ref[sample], dt, "c6 per-request plans")
    log(f"  per-request max|err|={stats['max_abs']:.3g} mean|err|={stats['mean_abs']:.3g}")
