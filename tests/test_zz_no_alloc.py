"""pa_decode_noalloc: pa_decode with the library's built-in scratch array as
its workspace, for callers that cannot allocate device memory.

It must write exactly what pa_decode writes with a caller workspace (same
kernels, same plan, so bitwise), on two calls in a row where the second has
a smaller batch, and stay within the oracle's tolerance; the binding must
allocate nothing through torch either; and a plan whose workspace exceeds
the array must be refused before the device is touched."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from flows import (assert_close, bits, oracle_decode_step, plan_and_workspace, product_decode_step, to_dev, to_host)


@pytest.fixture(scope="module")
def pk():
    import paged_kv_cache_115_amd as m
    return m


def _run_both(pk, pool, q_dev, tables, lens, scale, schedule, new_rows=None):
    hkv, hq, d = pool.k.shape[2], q_dev.shape[1], pool.k.shape[3]
    plan, plan_dev, ws = plan_and_workspace(pk, lens, hkv, hq, d, *schedule)
    assert plan.num_records > 0, "the schedule must cut sequences so that the workspace is used"
    assert pk.decode_workspace_bytes(plan, hq, d) <= pk._lib.PA_NOALLOC_SCRATCH_BYTES
    nk, nv = new_rows if new_rows is not None else (None, None)
    td, ld = to_dev(tables), to_dev(lens)
    want = torch.full(tuple(q_dev.shape), float("nan"), dtype=torch.float32, device="cuda")
    pk.decode(pool, q_dev, td, ld, scale, plan, plan_dev, ws, out=want, new_key=nk, new_value=nv)
    got = torch.full(tuple(q_dev.shape), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    pk.decode_noalloc(pool, q_dev, td, ld, scale, plan, plan_dev, got, new_key=nk, new_value=nv)
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    torch.cuda.synchronize()
    assert after == before, "decode_noalloc allocated device memory through torch"
    return to_host(got), to_host(want)


@pytest.mark.gpu
@pytest.mark.parametrize("name,schedule", [("c3s", (None, 1)), ("c3s", (7, 3)), ("c1", (None, 1))])
def test_noalloc_matches_workspace_decode_on_two_calls(pk, name, schedule):
    """Two calls in a row on one device, the second over the first half of
    the batch (a smaller plan, fewer records): both bitwise equal to pa_decode
    with a caller workspace, and within tolerance of the oracle."""
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    print(f"noalloc {name} schedule={schedule}", flush=True)
    case = synth.decode_case(name)
    dt = case["cfg"]["dtype"]
    step = product_decode_step(pk, case, schedule)
    ref = oracle_decode_step(case)
    got, want = _run_both(pk, step["pool"], step["q_dev"], step["tables"], step["lens"], case["scale"], schedule)
    assert np.array_equal(bits(got), bits(want))
    assert_close(got, ref["out"], dt, f"noalloc {name} first call")
    half = max(1, len(step["lens"]) // 2)
    got2, want2 = _run_both(pk, step["pool"], step["q_dev"][:half].contiguous(), step["tables"][:half],
                            step["lens"][:half], case["scale"], schedule)
    assert np.array_equal(bits(got2), bits(want2))
    assert_close(got2, ref["out"][:half], dt, f"noalloc {name} second, smaller call")


@pytest.mark.gpu
def test_noalloc_with_the_append_fused(pk):
    """The bench step's form (new rows fused into the call), twice in a row."""
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    case = synth.decode_case("c3s")
    step = product_decode_step(pk, case, (None, 1))
    ref = oracle_decode_step(case)
    off, lens = case["offsets"], step["lens"]
    last = np.array([off[s + 1] - 1 if lens[s] > 0 else 0 for s in range(len(lens))])
    rows = (to_dev(case["keys"][last]), to_dev(case["values"][last]))
    for _ in range(2):
        got, want = _run_both(pk, step["pool"], step["q_dev"], step["tables"], lens, case["scale"], (None, 1), rows)
        assert np.array_equal(bits(got), bits(want))
        assert_close(got, ref["out"], "bf16", "noalloc fused")
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(step["pool"].k)), bits(ref["kpool"]))
    assert np.array_equal(bits(to_host(step["pool"].v)), bits(ref["vpool"]))


def test_noalloc_refuses_a_plan_larger_than_its_scratch(pk):
    """Checked from the plan's info alone, before any device call: runs on a
    host without a GPU too."""
    lens = np.full(64, 4096, dtype=np.int32)
    plan = pk.decode_plan(lens, 8, num_workgroups=512, max_piece_tiles=1)
    need = pk.decode_workspace_bytes(plan, 32, 128)
    assert need > pk._lib.PA_NOALLOC_SCRATCH_BYTES
    pool = pk._lib.PaKvPool(0x10000, 0x20000, 100, 16, 8, 128, 1)
    p = ctypes.c_void_p(0x40000)
    st = pk._lib.lib.pa_decode_noalloc(ctypes.byref(pool), p, p, 0, p, 256, p, 64, 32, ctypes.c_float(0.1), None,
                                       None, p, ctypes.byref(plan.info), None)
    assert st == -1
    assert b"built-in scratch" in pk._lib.lib.pa_last_error()
