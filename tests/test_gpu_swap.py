"""GPU parity of swapping: pa_swap_blocks against the oracle's byte copy
(bit-exact, both directions, both engines), and a decode run that outgrows its
pool, preempting sequences to pinned host memory and bringing them back, run
through the library and through the oracle side by side."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth

from flows import _OracleSide, _ProductSide, assert_close, bits, preempt_run, to_dev, to_host, to_pinned

pytestmark = pytest.mark.gpu

ENGINES = ["kernel", "memcpy"]


@pytest.fixture(scope="module")
def pk():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import paged_kv_cache_115_amd as m
    return m


def _engine(pk, name):
    return pk.PA_SWAP_ENGINE_KERNEL if name == "kernel" else pk.PA_SWAP_ENGINE_MEMCPY


def _pairs(rng, n, n_src, n_dst, run):
    """n (src, dst) pairs with distinct destinations: a leading run of `run`
    consecutive ids on both sides (one runtime copy per pool), the rest scattered."""
    src = rng.choice(n_src, size=n, replace=True)
    dst = rng.permutation(n_dst)[:n]
    s0, d0 = int(rng.integers(0, n_src - run)), int(rng.integers(0, n_dst - run))
    run_dst = np.arange(d0, d0 + run)
    rest = dst[~np.isin(dst, run_dst)][: n - run]
    src[:run] = np.arange(s0, s0 + run)
    return np.stack([src, np.concatenate([run_dst, rest])], axis=1).astype(np.int32)


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("dt,b,hkv,d,n", [("bf16", 16, 8, 128, 261), ("bf16", 32, 2, 128, 17),
                                          ("f32", 8, 4, 64, 500), ("bf16", 8, 8, 128, 1)])
def test_swap_blocks_bit_exact(pk, engine, dt, b, hkv, d, n):
    print(f"swap_blocks engine={engine} dt={dt} B={b} Hkv={hkv} D={d} pairs={n}", flush=True)
    rng = np.random.default_rng(40 + n)
    nb, nh = 600, 520
    shape, hshape = (nb, b, hkv, d), (nh, b, hkv, d)
    kp, vp = synth.byte_pattern(shape, dt, 7), synth.byte_pattern(shape, dt, 8)
    hk, hv = synth.byte_pattern(hshape, dt, 9), synth.byte_pattern(hshape, dt, 10)
    kd, vd = to_dev(kp), to_dev(vp)
    hkt, hvt = to_pinned(hk), to_pinned(hv)
    pool, host = pk.KvPool(kd, vd), pk.HostKvPool(hkt, hvt)
    eng = _engine(pk, engine)

    out_pairs = _pairs(rng, n, nb, nh, min(n, 9))
    pk.swap_blocks(pool, host, out_pairs, pk.PA_SWAP_OUT, eng)
    pk.swap_blocks(pool, host, np.zeros((0, 2), np.int32), pk.PA_SWAP_OUT, eng)   # no-op
    torch.cuda.synchronize()
    oracle.swap_blocks(kp, vp, hk, hv, out_pairs)
    assert np.array_equal(bits(to_host(hkt)), bits(hk))
    assert np.array_equal(bits(to_host(hvt)), bits(hv))

    in_pairs = _pairs(rng, n, nh, nb, min(n, 5))
    pk.swap_blocks(pool, host, in_pairs, pk.PA_SWAP_IN, eng)
    torch.cuda.synchronize()
    oracle.swap_blocks(hk, hv, kp, vp, in_pairs)
    assert np.array_equal(bits(to_host(kd)), bits(kp))
    assert np.array_equal(bits(to_host(vd)), bits(vp))


def test_swap_rejects_unpinned_host_memory(pk):
    dev = torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    pool = pk.KvPool(dev, dev.clone())
    plain = torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pk.HostKvPool(plain, plain.clone())
    # Straight through the C ABI: pageable memory is refused before any copy,
    # and the refusal leaves no error behind for the next launch.
    from paged_kv_cache_115_amd import _lib
    plain_v = plain.clone()
    host = _lib.PaKvPool(plain.data_ptr(), plain_v.data_ptr(), 4, 16, 8, 128, 1)
    pairs = np.array([[0, 1]], dtype=np.int32)
    st = _lib.lib.pa_swap_blocks(ctypes.byref(pool.c), ctypes.byref(host),
                                 pairs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1, 0, 0, None)
    assert st == -1 and b"pinned" in _lib.lib.pa_last_error()
    # Host pool passed as the device pool: refused as well.
    pinned = plain.pin_memory()
    hp = pk.HostKvPool(pinned, plain.clone().pin_memory())
    st = _lib.lib.pa_swap_blocks(ctypes.byref(hp.c), ctypes.byref(hp.c),
                                 pairs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1, 0, 0, None)
    assert st == -1
    pk.copy_blocks(pool, to_dev(np.array([[0, 1]], np.int32)))
    torch.cuda.synchronize()


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("name", ["p1s", "p1f"])
def test_preemption_run_matches_oracle(pk, engine, name):
    print(f"preemption run {name} engine={engine}", flush=True)
    case = synth.preempt_case(name)
    dt = case["cfg"]["dtype"]
    ref = _OracleSide(case)
    o_log, o_out, o_tables, o_running = preempt_run(ref, case)
    side = _ProductSide(pk, case, _engine(pk, engine))
    p_log, p_out, p_tables, p_running = preempt_run(side, case)
    assert p_log == o_log and p_running == o_running
    assert any(e[1] == "out" for e in o_log) and any(e[1] == "in" for e in o_log)
    assert np.array_equal(p_tables, o_tables)
    assert_close(p_out, o_out, dt, f"{name}/{engine}")
    assert np.array_equal(bits(to_host(side.kd)), bits(ref.k))
    assert np.array_equal(bits(to_host(side.vd)), bits(ref.v))
    assert np.array_equal(bits(to_host(side.hk)), bits(ref.hk))
    assert np.array_equal(bits(to_host(side.hv)), bits(ref.hv))
