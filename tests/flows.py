"""End-to-end flows used by the GPU parity tests.

Each flow runs twice on the same seeded inputs from `synth`:
  * product path: the library's C++ block manager hands out blocks and slots,
    pa_copy_blocks / pa_reshape_and_cache fill a device pool whose unused
    slots hold NaN, pa_decode attends through the exported tables;
  * oracle path: the Python block-manager model, numpy byte copies and the
    float64 attention oracle.
Tables, slots and copy pairs must match exactly; pools bit-exactly; outputs
within the stated tolerance.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

# Tolerances from the target statement: fp32 max |err| <= 1e-5; bf16 KV with
# fp32 accumulation max |err| <= 1e-2 and mean |err| <= 1e-3.
TOL = {"f32": dict(max_abs=1e-5, mean_abs=None), "bf16": dict(max_abs=1e-2, mean_abs=1e-3)}


def torch_dtype(dt: str):
    return torch.float32 if dt == "f32" else torch.bfloat16


def to_dev(a: np.ndarray, dt: str | None = None) -> torch.Tensor:
    """Host array -> device tensor; uint16 arrays are bfloat16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def assert_close(out: np.ndarray, ref: np.ndarray, dt: str, where: str = "") -> dict:
    err = np.abs(out.astype(np.float64) - ref)
    stats = dict(max_abs=float(err.max()) if err.size else 0.0, mean_abs=float(err.mean()) if err.size else 0.0)
    tol = TOL[dt]
    assert np.all(np.isfinite(out)), f"{where}: non-finite output"
    assert stats["max_abs"] <= tol["max_abs"], f"{where}: max |err| {stats['max_abs']:.3g} > {tol['max_abs']}"
    if tol["mean_abs"] is not None:
        assert stats["mean_abs"] <= tol["mean_abs"], f"{where}: mean |err| {stats['mean_abs']:.3g}"
    return stats


def plan_and_workspace(pk, lens: np.ndarray, hkv: int, hq: int, d: int, num_workgroups=None, max_piece_tiles=0,
                       shared_kv=False):
    plan = pk.decode_plan(lens, hkv, num_workgroups, max_piece_tiles, shared_kv=shared_kv)
    nbytes = pk.decode_workspace_bytes(plan, hq, d)
    # The workspace needs no initialisation: fill it with NaN to prove it.
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda") if nbytes else None
    return plan, plan.to_device(), ws


def gpu_decode(pk, pool, q_dev, tables, lens, scale, schedule=(None, 0), out_dtype=torch.float32, shared_kv=False,
               new_key=None, new_value=None):
    """schedule = (num_workgroups or None for the device default, max_piece_tiles).
    new_key/new_value: fuse this step's append into the decode call."""
    hq = q_dev.shape[1]
    plan, plan_dev, ws = plan_and_workspace(pk, lens, pool.k.shape[2], hq, pool.k.shape[3], *schedule,
                                            shared_kv=shared_kv)
    out = torch.full(tuple(q_dev.shape), float("nan"), dtype=out_dtype, device="cuda")
    pk.decode(pool, q_dev, to_dev(tables), to_dev(lens), scale, plan, plan_dev, ws, out=out,
              new_key=new_key, new_value=new_value)
    return out


# ---------------------------------------------------------------- decode step
def product_decode_step(pk, case: dict, schedule=(None, 0), out_dtype=torch.float32, fused: bool = False):
    """Prefill L-1 tokens, append this step's token, decode.  Returns dict.
    fused: the appended token is not written by pa_reshape_and_cache but
    handed to pa_decode (new_key/new_value), which stores it while attending."""
    cfg = case["cfg"]
    b, hkv, d, dt = cfg["block_size"], cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    nb = case["num_blocks"]
    lens = case["lengths"]
    off = case["offsets"]
    s_count = len(lens)
    bm = pk.BlockManager(nb, b, case["free_order"])
    pre_slots, new_slots = [], []
    for s in range(s_count):
        sl, cw = bm.append(s, int(lens[s]) - 1 if lens[s] > 0 else 0)
        assert len(cw) == 0
        pre_slots.append(sl)
    for s in range(s_count):
        if lens[s] > 0:
            sl, cw = bm.append(s, 1)
            assert len(cw) == 0
            new_slots.append(int(sl[0]))
        else:
            new_slots.append(-1)
    bm.check()
    shape = (nb, b, hkv, d)
    kpool = to_dev(synth.nan_fill(shape, dt))
    vpool = to_dev(synth.nan_fill(shape, dt))
    pool = pk.KvPool(kpool, vpool)
    # Prefill rows: every token but the last of each sequence.
    pre_rows = np.concatenate([np.arange(off[s], off[s + 1] - 1) for s in range(s_count) if lens[s] > 0] or [np.zeros(0, np.int64)])
    pre_slot_arr = np.concatenate([p for p in pre_slots] or [np.zeros(0, np.int64)]).astype(np.int64)
    if pre_rows.size:
        pk.reshape_and_cache(pool, to_dev(case["keys"][pre_rows]), to_dev(case["values"][pre_rows]), to_dev(pre_slot_arr))
    last_rows = np.array([off[s + 1] - 1 if lens[s] > 0 else 0 for s in range(s_count)])
    new_k, new_v = to_dev(case["keys"][last_rows]), to_dev(case["values"][last_rows])
    if not fused:
        pk.reshape_and_cache(pool, new_k, new_v, to_dev(np.array(new_slots, dtype=np.int64)))
    maxb = max(1, int(max((-(-int(L) // b)) for L in lens)))
    tables, lens_out = bm.export(np.arange(s_count), maxb)
    assert np.array_equal(lens_out, lens)
    out = gpu_decode(pk, pool, to_dev(case["q"]), tables, lens_out, case["scale"], schedule, out_dtype,
                     new_key=new_k if fused else None, new_value=new_v if fused else None)
    torch.cuda.synchronize()
    return dict(out=to_host(out), kpool=to_host(kpool), vpool=to_host(vpool), tables=tables,
                pre_slots=pre_slots, new_slots=new_slots, pool=pool, q_dev=to_dev(case["q"]), lens=lens_out)


def oracle_decode_step(case: dict, seqs=None):
    cfg = case["cfg"]
    b, hkv, d, dt = cfg["block_size"], cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    nb = case["num_blocks"]
    lens = case["lengths"]
    off = case["offsets"]
    bm = oracle.BlockManagerModel(nb, b, case["free_order"])
    shape = (nb, b, hkv, d)
    kpool = synth.nan_fill(shape, dt)
    vpool = synth.nan_fill(shape, dt)
    pre_slots, new_slots = [], []
    for s in range(len(lens)):
        sl, _ = bm.append(s, max(int(lens[s]) - 1, 0))
        pre_slots.append(np.array(sl, dtype=np.int64))
        oracle.reshape_and_cache(kpool, vpool, case["keys"][off[s]:off[s] + len(sl)],
                                 case["values"][off[s]:off[s] + len(sl)], np.array(sl, dtype=np.int64))
    for s in range(len(lens)):
        if lens[s] > 0:
            sl, _ = bm.append(s, 1)
            new_slots.append(sl[0])
            oracle.reshape_and_cache(kpool, vpool, case["keys"][off[s + 1] - 1:off[s + 1]],
                                     case["values"][off[s + 1] - 1:off[s + 1]], np.array(sl, dtype=np.int64))
        else:
            new_slots.append(-1)
    bm.check()
    maxb = max(1, int(max((-(-int(L) // b)) for L in lens)))
    tables = np.zeros((len(lens), maxb), dtype=np.int32)
    for s in range(len(lens)):
        t = bm.table(s)
        tables[s, :len(t)] = t
    out = oracle.decode_attention(case["q"], kpool, vpool, tables, lens, case["scale"], seqs=seqs)
    return dict(out=out, kpool=kpool, vpool=vpool, tables=tables, pre_slots=pre_slots, new_slots=new_slots)


# ------------------------------------------------------- prefix sharing (CoW)
def _prefix_ops(case: dict):
    """The operation script shared by both sides: prompts, forks, tails."""
    p, n = case["cfg"]["num_prompts"], case["cfg"]["samples"]
    return p, n, case["cfg"]["prefix_len"], case["tail_lengths"]


def cascade_decode(pk, pool, q_dev, tables, lens, scale, bm, seqs, schedule=(None, 0), new_key=None, new_value=None):
    """pa_decode over a plan that reads each shared prefix once per group
    (pa_bm_prefix_groups -> pa_decode_plan_prefix)."""
    hq = q_dev.shape[1]
    group, tokens = bm.prefix_groups(seqs)
    plan = pk.decode_plan_prefix(lens, pool.k.shape[2], hq, group, tokens, schedule[0], schedule[1])
    nbytes = pk.decode_workspace_bytes(plan, hq, pool.k.shape[3])
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda") if nbytes else None
    out = torch.full(tuple(q_dev.shape), float("nan"), dtype=torch.float32, device="cuda")
    pk.decode(pool, q_dev, to_dev(tables), to_dev(lens), scale, plan, plan.to_device(), ws, out=out,
              new_key=new_key, new_value=new_value)
    return out, plan


def product_prefix(pk, case: dict, schedule=(None, 0), shared: bool = True, private_order=None,
                   cascade: bool = False):
    cfg = case["cfg"]
    b, hkv, d, dt = case["block_size"], cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    p, n, pre, tails = _prefix_ops(case)
    nseq = p * n
    if shared:
        nb, order = case["num_blocks"], case["free_order"]
    else:
        nb = int(1.25 * (nseq * pre + int(tails.sum())) // b) + 2 * nseq + 1
        order = private_order if private_order is not None else np.arange(nb)
    bm = pk.BlockManager(nb, b, order)
    shape = (nb, b, hkv, d)
    kpool = to_dev(synth.nan_fill(shape, dt))
    vpool = to_dev(synth.nan_fill(shape, dt))
    pool = pk.KvPool(kpool, vpool)
    all_cows = []
    if shared:
        for i in range(p):
            parent = 1_000_000 + i
            sl, _ = bm.append(parent, pre)
            pk.reshape_and_cache(pool, to_dev(case["prefix_keys"][i]), to_dev(case["prefix_values"][i]), to_dev(sl))
            for j in range(n):
                bm.fork(parent, i * n + j)
            bm.free(parent)
    else:
        for i in range(p):
            for j in range(n):
                sl, _ = bm.append(i * n + j, pre)
                pk.reshape_and_cache(pool, to_dev(case["prefix_keys"][i]), to_dev(case["prefix_values"][i]), to_dev(sl))
    # First divergent token of every sample: copy-on-write, then the write.
    slots, cows = bm.append_step(np.arange(nseq))
    all_cows.append(cows)
    if len(cows):
        pk.copy_blocks(pool, to_dev(np.ascontiguousarray(cows, dtype=np.int32)))
    to = case["tail_offsets"]
    first = to[:-1]
    pk.reshape_and_cache(pool, to_dev(case["tail_keys"][first]), to_dev(case["tail_values"][first]), to_dev(slots))
    for s in range(nseq):
        if tails[s] > 1:
            sl, cw = bm.append(s, int(tails[s]) - 1)
            assert len(cw) == 0
            rows = np.arange(to[s] + 1, to[s + 1])
            pk.reshape_and_cache(pool, to_dev(case["tail_keys"][rows]), to_dev(case["tail_values"][rows]), to_dev(sl))
    bm.check()
    lens = (pre + tails).astype(np.int32)
    maxb = int(max(-(-int(L) // b) for L in lens))
    tables, lens_out = bm.export(np.arange(nseq), maxb)
    assert np.array_equal(lens_out, lens)
    stats = bm.stats()
    plan = None
    if cascade:
        out, plan = cascade_decode(pk, pool, to_dev(case["q"]), tables, lens, case["scale"], bm, np.arange(nseq),
                                   schedule)
    else:
        out = gpu_decode(pk, pool, to_dev(case["q"]), tables, lens, case["scale"], schedule,
                         shared_kv=stats["shared_blocks"] > 0)
    torch.cuda.synchronize()
    return dict(out=to_host(out), tables=tables, cows=np.concatenate(all_cows) if all_cows else None,
                stats=stats, pool=pool, lens=lens, kpool=kpool, vpool=vpool, bm=bm, plan=plan)


def oracle_prefix(case: dict, seqs=None):
    cfg = case["cfg"]
    b, hkv, d, dt = case["block_size"], cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    p, n, pre, tails = _prefix_ops(case)
    nseq = p * n
    nb = case["num_blocks"]
    bm = oracle.BlockManagerModel(nb, b, case["free_order"])
    shape = (nb, b, hkv, d)
    kpool = synth.nan_fill(shape, dt)
    vpool = synth.nan_fill(shape, dt)
    for i in range(p):
        parent = 1_000_000 + i
        sl, _ = bm.append(parent, pre)
        oracle.reshape_and_cache(kpool, vpool, case["prefix_keys"][i], case["prefix_values"][i], np.array(sl))
        for j in range(n):
            bm.fork(parent, i * n + j)
        bm.free_seq(parent)
    slots, cows = bm.append_step(range(nseq))
    oracle.copy_blocks(kpool, vpool, np.array(cows, dtype=np.int64).reshape(-1, 2))
    to = case["tail_offsets"]
    first = to[:-1]
    oracle.reshape_and_cache(kpool, vpool, case["tail_keys"][first], case["tail_values"][first], np.array(slots))
    for s in range(nseq):
        if tails[s] > 1:
            sl, _ = bm.append(s, int(tails[s]) - 1)
            rows = np.arange(to[s] + 1, to[s + 1])
            oracle.reshape_and_cache(kpool, vpool, case["tail_keys"][rows], case["tail_values"][rows], np.array(sl))
    bm.check()
    lens = (pre + tails).astype(np.int32)
    maxb = int(max(-(-int(L) // b) for L in lens))
    tables = np.zeros((nseq, maxb), dtype=np.int32)
    for s in range(nseq):
        t = bm.table(s)
        tables[s, :len(t)] = t
    out = oracle.decode_attention(case["q"], kpool, vpool, tables, lens, case["scale"], seqs=seqs)
    return dict(out=out, tables=tables, cows=np.array(cows, dtype=np.int32).reshape(-1, 2), stats=bm.stats(),
                kpool=kpool, vpool=vpool)
