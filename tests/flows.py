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
                       kind=-1, shared_kv=False, block_size=None):
    """kind: a pk.SCHEDULE_* value (-1, the default: the automatic choice).
    block_size: the pool's B (below 8 it caps the pieces)."""
    plan = pk.decode_plan(lens, hkv, num_workgroups, max_piece_tiles, shared_kv=shared_kv, schedule=kind,
                          block_size=block_size)
    nbytes = pk.decode_workspace_bytes(plan, hq, d)
    # The workspace needs no initialisation: fill it with NaN to prove it.
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda") if nbytes else None
    return plan, plan.to_device(), ws


def gpu_decode(pk, pool, q_dev, tables, lens, scale, schedule=(None, 0), out_dtype=torch.float32, shared_kv=False,
               new_key=None, new_value=None, first_blocks=False):
    """schedule = (num_workgroups or None for the device default, max_piece_tiles[, schedule kind]).
    new_key/new_value: fuse this step's append into the decode call.
    first_blocks: write the jobs' first-tile table entries into the plan."""
    hq = q_dev.shape[1]
    plan, plan_dev, ws = plan_and_workspace(pk, lens, pool.k.shape[2], hq, pool.k.shape[3], *schedule,
                                            shared_kv=shared_kv, block_size=pool.block_size)
    if first_blocks:
        plan.set_first_blocks(tables, pool.block_size)
        plan_dev = plan.to_device()
    out = torch.full(tuple(q_dev.shape), float("nan"), dtype=out_dtype, device="cuda")
    pk.decode(pool, q_dev, to_dev(tables), to_dev(lens), scale, plan, plan_dev, ws, out=out,
              new_key=new_key, new_value=new_value)
    return out


# ---------------------------------------------------------------- decode step
def product_decode_step(pk, case: dict, schedule=(None, 0), out_dtype=torch.float32, fused: bool = False,
                        first_blocks: bool = False):
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
                     new_key=new_k if fused else None, new_value=new_v if fused else None, first_blocks=first_blocks)
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


def cascade_decode(pk, pool, q_dev, tables, lens, scale, bm, seqs, schedule=(None, 0), new_key=None, new_value=None,
                   first_blocks=False):
    """pa_decode over a plan that reads each shared prefix once per group
    (pa_bm_prefix_groups -> pa_decode_plan_prefix)."""
    hq = q_dev.shape[1]
    group, tokens = bm.prefix_groups(seqs)
    plan = pk.decode_plan_prefix(lens, pool.k.shape[2], hq, group, tokens, schedule[0], schedule[1],
                                 block_size=pool.block_size)
    if first_blocks:
        plan.set_first_blocks(tables, pool.block_size)
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


# ------------------------------------------------------------- preemption
class _OracleSide:
    """Python block-manager model, numpy pools and byte copies."""

    def __init__(self, case):
        cfg = case["cfg"]
        self.b, dt = cfg["block_size"], cfg["dtype"]
        shape = (case["num_blocks"], self.b, cfg["num_kv_heads"], cfg["head_dim"])
        hshape = (case["host_blocks"],) + shape[1:]
        self.bm = oracle.BlockManagerModel(case["num_blocks"], self.b, case["free_order"])
        self.bm.set_host_blocks(case["host_blocks"])
        self.k, self.v = synth.nan_fill(shape, dt), synth.nan_fill(shape, dt)
        self.hk, self.hv = synth.nan_fill(hshape, dt), synth.nan_fill(hshape, dt)

    def append(self, seqs, n=1):
        """n tokens for one sequence (n given) or one token for each of seqs."""
        try:
            slots, cows = self.bm.append(seqs[0], n) if len(seqs) == 1 and n != 1 else self.bm.append_step(seqs)
        except oracle.OutOfBlocks:
            return None
        if cows:
            oracle.copy_blocks(self.k, self.v, np.array(cows))
        return np.array(slots, dtype=np.int64)

    def write(self, slots, rk, rv):
        oracle.reshape_and_cache(self.k, self.v, rk, rv, slots)

    def swap(self, seqs, out):
        try:
            pairs = self.bm.swap_out(seqs) if out else self.bm.swap_in(seqs)
        except oracle.OutOfBlocks:
            return None
        if out:
            oracle.swap_blocks(self.k, self.v, self.hk, self.hv, np.array(pairs))
        else:
            oracle.swap_blocks(self.hk, self.hv, self.k, self.v, np.array(pairs))
        return [tuple(p) for p in pairs]

    def fork(self, p, c):
        self.bm.fork(p, c)

    def free(self, s):
        self.bm.free_seq(s)

    def free_blocks(self):
        return len(self.bm.free)

    def table_len(self, s):
        return len(self.bm.table(s))

    def decode(self, seqs, q, scale):
        maxb = max(1, max(self.table_len(s) for s in seqs))
        tables = np.zeros((len(seqs), maxb), dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self.bm.table(s)
            tables[i, :len(t)] = t
        lens = np.array([self.bm.length(s) for s in seqs], dtype=np.int32)
        self.bm.check()
        return oracle.decode_attention(q, self.k, self.v, tables, lens, scale), tables


class _ProductSide:
    """The library: C++ block manager, device pools, pinned host pools."""

    def __init__(self, pk, case, engine):
        cfg = case["cfg"]
        self.pk, self.engine = pk, engine
        self.b, dt = cfg["block_size"], cfg["dtype"]
        shape = (case["num_blocks"], self.b, cfg["num_kv_heads"], cfg["head_dim"])
        hshape = (case["host_blocks"],) + shape[1:]
        self.bm = pk.BlockManager(case["num_blocks"], self.b, case["free_order"])
        self.bm.set_host_blocks(case["host_blocks"])
        self.kd, self.vd = to_dev(synth.nan_fill(shape, dt)), to_dev(synth.nan_fill(shape, dt))
        self.pool = pk.KvPool(self.kd, self.vd)
        self.hk, self.hv = to_pinned(synth.nan_fill(hshape, dt)), to_pinned(synth.nan_fill(hshape, dt))
        self.host = pk.HostKvPool(self.hk, self.hv)

    def append(self, seqs, n=1):
        try:
            slots, cows = self.bm.append(seqs[0], n) if len(seqs) == 1 and n != 1 else self.bm.append_step(seqs)
        except self.pk.PaError as e:
            assert e.status == -3, e
            return None
        if len(cows):
            self.pk.copy_blocks(self.pool, to_dev(cows))
        return slots

    def write(self, slots, rk, rv):
        self.pk.reshape_and_cache(self.pool, to_dev(rk), to_dev(rv), to_dev(slots))

    def swap(self, seqs, out):
        try:
            pairs = self.bm.swap_out(seqs) if out else self.bm.swap_in(seqs)
        except self.pk.PaError as e:
            assert e.status == -3, e
            return None
        self.pk.swap_blocks(self.pool, self.host, pairs, self.pk.PA_SWAP_OUT if out else self.pk.PA_SWAP_IN,
                            self.engine)
        return [tuple(p) for p in pairs.tolist()]

    def fork(self, p, c):
        self.bm.fork(p, c)

    def free(self, s):
        self.bm.free(s)

    def free_blocks(self):
        return self.bm.stats()["free_blocks"]

    def table_len(self, s):
        return len(self.bm.table(s))

    def decode(self, seqs, q, scale):
        maxb = max(1, max(self.table_len(s) for s in seqs))
        tables, lens = self.bm.export(seqs, maxb)
        self.bm.check()
        out = gpu_decode(self.pk, self.pool, to_dev(q), tables, lens, scale)
        torch.cuda.synchronize()
        return to_host(out), tables


def to_pinned(a: np.ndarray) -> torch.Tensor:
    """Host array -> pinned host tensor; uint16 arrays are bfloat16 bit patterns."""
    t = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16) if a.dtype == np.uint16 \
        else torch.from_numpy(np.ascontiguousarray(a).copy())
    return t.pin_memory()


def preempt_run(side, case: dict):
    """A decode run that outgrows its pool, identical on both sides.

    Policy (a scheduler's choice; the pages leave it open): prompts are
    prefilled in order, then sequence 0 is forked into its samples, which
    join the end of the running list; each step first swaps the oldest
    swapped sequence back in if its table plus one block per running
    sequence fits in the free list, then appends one token to every running
    sequence; when that does not fit, the most recently admitted running
    sequence is swapped out alone and the step is retried.  At step
    `group_out_at` the two most recently admitted running sequences are
    swapped out together; at the `retire_at` steps the oldest running
    sequence retires.  At the end all swapped sequences come back in one call
    (retiring the oldest runners until they fit) and every running sequence
    is decoded.  Returns (event log, output, tables,
    running sequence ids)."""
    cfg = case["cfg"]
    s_count, samples = cfg["num_seqs"], cfg["samples"]
    cursor = 0

    def rows(n):
        nonlocal cursor
        r = slice(cursor, cursor + n)
        cursor += n
        return case["rows_k"][r], case["rows_v"][r]

    log_ = []
    running, swapped = [], []
    for s in range(s_count):
        n = int(case["prompts"][s])
        slots = side.append([s], n)
        assert slots is not None, "prompts are sized to fit the pool"
        side.write(slots, *rows(n))
        running.append(s)
    for j in range(1, samples):
        side.fork(0, s_count + j - 1)
        running.append(s_count + j - 1)
    for step in range(cfg["steps"]):
        if step == cfg["group_out_at"] and len(running) >= 2:
            group = running[-2:]
            pairs = side.swap(group, out=True)
            assert pairs is not None, "host pool is sized to hold every victim"
            log_.append((step, "out", tuple(group), pairs))
            del running[-2:]
            swapped.extend(group)
        if swapped and side.free_blocks() >= side.table_len(swapped[0]) + len(running) + 1:
            pairs = side.swap([swapped[0]], out=False)
            if pairs is not None:
                log_.append((step, "in", swapped[0], pairs))
                running.append(swapped.pop(0))
        while running:
            slots = side.append(running)
            if slots is not None:
                break
            victim = running.pop()
            pairs = side.swap([victim], out=True)
            assert pairs is not None, "host pool is sized to hold every victim"
            log_.append((step, "out", victim, pairs))
            swapped.append(victim)
        if running:
            side.write(slots, *rows(len(running)))
        if step in cfg["retire_at"] and running:
            log_.append((step, "retire", running[0], []))
            side.free(running.pop(0))
    while swapped:
        pairs = side.swap(swapped, out=False)
        if pairs is None:
            log_.append(("end", "retire", running[0], []))
            side.free(running.pop(0))
            continue
        log_.append(("end", "in", tuple(swapped), pairs))
        running.extend(swapped)
        swapped = []
    q = case["q"][np.array(running)]
    out, tables = side.decode(running, q, case["scale"])
    return log_, out, tables, running
