#!/usr/bin/env python3
"""Benchmark: paged decode attention on one MI355X.

Workload (default): GQA decode in bf16, batch 256, 32 query heads over 8 KV
heads (group 4), head_dim 128, block size 16, context lengths lognormal with
mean about 200 tokens capped at 4096, blocks handed out from a shuffled free
list.  One step is one pass of the whole hot path over one batch:
  pa_copy_blocks (copy-on-write pairs of this step; none in this workload)
  -> pa_decode with this step's new keys and values: the attention launch
     (through the block tables, on a persistent grid) takes every sequence's
     token L - 1 from them, and the merge launch (cut sequences) stores that
     token into its slot, which is pa_reshape_and_cache's work, fused.
The same step as three calls (pa_copy_blocks -> pa_reshape_and_cache ->
pa_decode without new keys/values) is timed too (ms_per_step_eager).
Step inputs (tables, lengths, slots, the decode plan, queries, new keys and
values) are resident in device memory before timing; the host block-manager
append and the host plan that produce them are timed separately
(host_append_us; host_plan_us, the median of warm plan builds).  R pool replicas (>= 1 GiB together, four
times the 256 MB last-level cache) rotate so that KV reads come from HBM.

Prints one JSON line.  `value` is KV-read GB/s over whole steps: algorithmic KV
bytes (each live token's K and V row of each KV head, read once) per step
divided by the step time.  `roofline` reports the step's attention launch
alone (append fused): the same algorithmic bytes over its average launch time,
from HIP events on the stream the launches run on around K back-to-back
attention launches (a second timed region after the steps; pa_decode is issued
as its two launches, pa_decode_attention and pa_decode_merge_pieces, for
this).  The launch without the fused append (as in the three-call step) is
timed the same way (attention_launch_unfused_us, unfused_frac).
"""
from __future__ import annotations

import os

for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = "1"   # the CPU baseline is single-threaded by design

import argparse
import hashlib
import json
import math
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
WORKLOADS = {
    "c3": "GQA decode bf16: batch 256, 32 q heads / 8 KV heads, head_dim 128, block 16, "
          "lognormal lengths (mean ~200, cap 4096), shuffled blocks",
    "c3f": "GQA decode fp32: batch 256, 32 q heads / 8 KV heads, head_dim 128, block 16, "
           "lognormal lengths (mean ~200, cap 4096), shuffled blocks (the c3 batch in fp32)",
    "c2": "MHA decode bf16: batch 64, 32/32 heads, head_dim 128, block 16, lengths U[1,2048]",
    "c4": "long-context GQA decode bf16: batch 16, 64 q / 8 KV heads, head_dim 128, block 16, "
          "lengths U[16384,32768]",
    "c5": "prefix sharing bf16: 32 prompts x 4 samples sharing a 2000-token prefix, private tails U[1,512], "
          "32 q / 8 KV heads, head_dim 128; the step where the samples diverge",
    "c6": "prefix cache across requests bf16: 256 requests opening with one of 4 shared 2000-token system "
          "prompts, private user turns U[1,400], 32 q / 8 KV heads, head_dim 128; admitted through the prefix "
          "cache, decoded with the cascade plan",
}
PMC_FILE = os.path.join(ROOT, "profiles", "decode_c3_pmc.json")
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_115_amd", "csrc", "decode_kernels.hip")


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic(config: str, schedule: list):
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel source and this workload."""
    try:
        rec = json.load(open(PMC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_hash() or rec.get("config") != config or rec.get("schedule") != schedule:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(case, per_token: int, k_host, v_host, tables, lens, budget_s: float):
    """The float64 oracle over the sequences of the same batch, in order and
    wrapping around, until about `budget_s` seconds of single-core work;
    reported in the headline unit (KV GB/s, `per_token` bytes per context
    token) and as sequences per second."""
    import oracle
    t0 = time.perf_counter()
    done, tokens = 0, 0
    while time.perf_counter() - t0 < budget_s:
        s = done % len(lens)
        oracle.decode_attention(case["q"], k_host, v_host, tables, lens, case["scale"], seqs=[s])
        tokens += int(lens[s])
        done += 1
    dt = time.perf_counter() - t0
    cores_total = len(os.sched_getaffinity(0))
    return {"value": round(tokens * per_token / dt / 1e9, 6), "unit": "GB/s", "cores": 1, "cores_total": cores_total,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"float64 oracle, {done} sequence decodes cycling through the {len(lens)}-sequence batch "
                      f"({tokens} context tokens, {dt:.1f} s on 1 host core of {cores_total})",
            "seconds": round(dt, 3), "seqs_per_s": round(done / dt, 3)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def percentiles(xs) -> dict:
    a = np.asarray(xs, dtype=float)
    return {"p10": round(float(np.percentile(a, 10)), 3), "p50": round(float(np.percentile(a, 50)), 3),
            "p90": round(float(np.percentile(a, 90)), 3), "mean": round(float(a.mean()), 3)}


def read_probe(torch, pk, nbytes: int, reps: int = 50, workgroups: int = 512) -> dict:
    """pa_probe_read over nbytes, rotating through a buffer of at least
    1.25 GiB (five times the 256 MB last-level cache) so that every read comes
    from HBM; microseconds per launch from HIP events on the stream."""
    dev = torch.device("cuda", 0)
    span = max(nbytes, 256 << 20)
    regions = max(2, -(-(5 << 28) // span))
    buf = torch.ones(span * regions // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(workgroups * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    views = [buf[r * span // 4:(r * span + nbytes) // 4] for r in range(regions)]
    for i in range(5):
        pk.probe_read(views[i % regions], workgroups, sink, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        pk.probe_read(views[i % regions], workgroups, sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    del buf
    return {"bytes": nbytes, "workgroups": workgroups, "us": round(us, 3), "GBs": round(nbytes / us / 1e3, 1),
            "frac_of_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}


def read_probe_sweep(torch, pk) -> int:
    """The probe at 16 MB .. 1 GiB: a least-squares fit of launch time against
    bytes gives the fixed cost of a launch and the streaming rate."""
    rows = [read_probe(torch, pk, n) for n in (16 << 20, 64 << 20, 220954624, 512 << 20, 1 << 30)]
    x = np.array([r["bytes"] for r in rows], float)
    y = np.array([r["us"] for r in rows], float)
    slope, fixed = np.polyfit(x, y, 1)
    print(json.dumps({"metric": "streaming read (pa_probe_read) time against bytes", "fixed_us": round(float(fixed), 2),
                      "streaming_GBs": round(float(1e3 / (slope * 1e9) * 1e3), 1),
                      "streaming_frac_of_peak": round(float(1e3 / (slope * 1e9) * 1e3) / HBM_PEAK_GBS, 4),
                      "config": {"workload": "one contiguous read per launch, 512 workgroups of 256 threads, "
                                             "16-byte non-temporal loads"}, "sweep": rows}), flush=True)
    return 0


def decode_workload(pk, name: str, block_size: int | None = None) -> dict:
    """One decode step of a named workload: every sequence holds L - 1
    tokens; the step appends one token to each (timed host append) and
    attends over L.  block_size overrides the workload's block size (same
    lengths; a pool of the same slack and a seeded shuffled free list)."""
    case = synth.decode_case(name)
    cfg = case["cfg"]
    lens_np = case["lengths"]
    S, B = len(lens_np), cfg["block_size"]
    if block_size is not None and block_size != B:
        B = block_size
        nb = synth.pool_blocks_for(lens_np, B)
        case = dict(case, num_blocks=nb, free_order=np.random.default_rng(cfg["seed"] + 100 * B).permutation(nb).astype(np.int32))
    bm = pk.BlockManager(case["num_blocks"], B, case["free_order"])
    for s in range(S):
        bm.append(s, int(lens_np[s]) - 1)
    seqs = np.arange(S)
    t0 = time.perf_counter()
    slots, cows = bm.append_step(seqs)
    host_append_us = (time.perf_counter() - t0) * 1e6
    maxb = int(max(-(-int(L) // B) for L in lens_np))
    tables, lens = bm.export(seqs, maxb)
    desc = WORKLOADS[name] if B == cfg["block_size"] else WORKLOADS[name].replace("block 16", f"block {B}")
    return dict(name=name, desc=desc, case=case, seed=cfg["seed"], S=S, hq=cfg["num_q_heads"],
                hkv=cfg["num_kv_heads"], d=cfg["head_dim"], B=B, nb=case["num_blocks"], tables=tables, lens=lens,
                slots=slots, cows=cows, host_append_us=host_append_us, unique_tokens=int(lens.sum()),
                shared_kv=bm.stats()["shared_blocks"] > 0, bm=bm)


def prefix_workload(pk, block_size: int) -> dict:
    """The step at which shared-prefix samples diverge.  Each prompt's prefix
    is written once and forked into its samples; every sample then holds its
    private tail but the last token.  The step: pa_copy_blocks with the
    copy-on-write pairs of the divergence (the shared partial block, once per
    sample but the last), pa_reshape_and_cache of every sample's last tail
    token, pa_decode over prefix + tail."""
    case = synth.prefix_case("c5", block_size)
    cfg = case["cfg"]
    p, n, pre, tails = cfg["num_prompts"], cfg["samples"], cfg["prefix_len"], case["tail_lengths"]
    B, nseq = block_size, p * n
    bm = pk.BlockManager(case["num_blocks"], B, case["free_order"])
    for i in range(p):
        parent = 1_000_000 + i
        bm.append(parent, pre)
        for j in range(n):
            bm.fork(parent, i * n + j)
        bm.free(parent)
    seqs = np.arange(nseq)
    fork_slots, fork_cows = bm.append_step(seqs)          # first divergent token: copy-on-write
    for s in range(nseq):
        if tails[s] > 2:
            bm.append(s, int(tails[s]) - 2)
    t0 = time.perf_counter()
    last = seqs[tails >= 2]
    slots = np.full(nseq, -1, dtype=np.int64)
    if last.size:
        sl, cw = bm.append_step(last)
        assert len(cw) == 0
        slots[last] = sl
    host_append_us = (time.perf_counter() - t0) * 1e6
    slots[tails == 1] = fork_slots[tails == 1]
    lens_np = (pre + tails).astype(np.int32)
    maxb = int(max(-(-int(L) // B) for L in lens_np))
    tables, lens = bm.export(seqs, maxb)
    assert np.array_equal(lens, lens_np)
    # Distinct (block, slot) pairs the step reads: shared prefix slots once.
    used = {}
    for s in range(nseq):
        nblk = -(-int(lens[s]) // B)
        for j, blk in enumerate(tables[s, :nblk]):
            fill = B if j < nblk - 1 else int(lens[s]) - j * B
            used[int(blk)] = max(used.get(int(blk), 0), fill)
    q = case["q"]
    group, prefix_tokens = bm.prefix_groups(seqs)
    return dict(name=f"c5 B={B}", desc=f"{WORKLOADS['c5']}, block {B}", case=dict(q=q, scale=case["scale"]),
                prefix_group=group, prefix_tokens=prefix_tokens,
                seed=cfg["seed"] + B, S=nseq, hq=cfg["num_q_heads"], hkv=cfg["num_kv_heads"], d=cfg["head_dim"], B=B,
                nb=case["num_blocks"], tables=tables, lens=lens, slots=slots,
                cows=np.asarray(fork_cows, dtype=np.int32).reshape(-1, 2), host_append_us=host_append_us,
                unique_tokens=int(sum(used.values())), shared_kv=bm.stats()["shared_blocks"] > 0, bm=bm)


def prefix_cache_workload(pk, block_size: int) -> dict:
    """Requests that share system prompts, admitted through the prefix cache
    (pa_bm_append_prompt: the second request of a system prompt onwards reuses
    its blocks), then one decode step: every request appends one token and
    attends over its prompt + 1.  Shared system-prompt blocks are read once per
    prefix group of the cascade plan."""
    case = synth.prefix_cache_case("c6")
    cfg = case["cfg"]
    prompts = case["prompts"]
    B, S = block_size, len(prompts)
    private_blocks = sum(-(-(len(p) + 1) // B) for p in prompts)
    nb = private_blocks + S
    bm = pk.BlockManager(nb, B, np.random.default_rng(cfg["seed"]).permutation(nb).astype(np.int32))
    bm.enable_prefix_cache()
    t0 = time.perf_counter()
    for r, p in enumerate(prompts):
        bm.append_prompt(r, p)
    host_prompt_us = (time.perf_counter() - t0) * 1e6 / S
    st = bm.stats()
    seqs = np.arange(S)
    t0 = time.perf_counter()
    slots, cows = bm.append_step(seqs)
    host_append_us = (time.perf_counter() - t0) * 1e6
    lens_np = np.array([len(p) + 1 for p in prompts], dtype=np.int32)
    maxb = int(max(-(-int(L) // B) for L in lens_np))
    tables, lens = bm.export(seqs, maxb)
    assert np.array_equal(lens, lens_np)
    used = {}
    for s in range(S):
        nblk = -(-int(lens[s]) // B)
        for j, blk in enumerate(tables[s, :nblk]):
            fill = B if j < nblk - 1 else int(lens[s]) - j * B
            used[int(blk)] = max(used.get(int(blk), 0), fill)
    group, prefix_tokens = bm.prefix_groups(seqs)
    desc = WORKLOADS["c6"] if B == 16 else WORKLOADS["c6"].replace("head_dim 128;", f"head_dim 128, block {B};")
    return dict(name="c6", desc=desc, case=dict(q=case["q"], scale=case["scale"]), prefix_group=group,
                prefix_tokens=prefix_tokens, seed=cfg["seed"], S=S, hq=cfg["num_q_heads"], hkv=cfg["num_kv_heads"],
                d=cfg["head_dim"], B=B, nb=nb, tables=tables, lens=lens, slots=slots,
                cows=np.asarray(cows, dtype=np.int32).reshape(-1, 2), host_append_us=host_append_us,
                unique_tokens=int(sum(used.values())), shared_kv=True, bm=bm,
                prefix_cache={"host_prompt_us_per_request": round(host_prompt_us, 2),
                              "prompt_tokens": int(st["prefix_query_tokens"]),
                              "reused_tokens": int(st["prefix_hit_tokens"]),
                              "prefill_tokens_to_compute": int(st["prefix_query_tokens"] - st["prefix_hit_tokens"]),
                              "blocks_held": int(st["used_blocks"]), "blocks_held_private": int(private_blocks - S),
                              "cached_blocks": int(st["cached_blocks"])})


def copy_blocks_probe(torch, pk, B: int, hkv: int, d: int, pairs: int = 4096, reps: int = 20) -> dict:
    """pa_copy_blocks on `pairs` random disjoint (src, dst) pairs of a pool of
    2 * pairs blocks, timed back to back; bytes = K and V, read and written."""
    nb = 2 * pairs
    dev = torch.device("cuda", 0)
    kp = torch.zeros((nb, B, hkv, d), dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    pool = pk.KvPool(kp, vp)
    perm = np.random.default_rng(9).permutation(nb).astype(np.int32)
    pr = torch.from_numpy(np.stack([perm[:pairs], perm[pairs:]], axis=1).copy()).to(dev)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        pk.copy_blocks(pool, pr, stream)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        pk.copy_blocks(pool, pr, stream)
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / reps * 1e3
    nbytes = pairs * 2 * B * hkv * d * 2 * 2
    return {"pairs": pairs, "block_size": B, "us": round(us, 2), "bytes": nbytes,
            "GBs": round(nbytes / us / 1e3, 1), "pct_hbm_peak": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 2)}


def copy_probe(torch, nbytes: int) -> int:
    """Device-to-device copy of nbytes (read nbytes, write nbytes): the
    runtime's copy kernel, timed, so that a counter run over this command
    gives the reading of a transfer of known size."""
    torch.cuda.set_device(0)
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    start.record()
    for _ in range(reps):
        b.copy_(a)
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / reps * 1e3
    print(json.dumps({"copy_bytes": a.numel() * 4, "calls": reps + 3, "us": round(us, 2),
                      "read_plus_write_GBs": round(2 * a.numel() * 4 / us / 1e3, 1)}), flush=True)
    return 0


def swap_sweep(torch, pk, lengths, reps: int = 10) -> int:
    """Preemption by swapping, one layer of the c3 head layout (8 KV heads,
    head_dim 128, bf16, block 16): a sequence of L tokens is swapped out to
    pinned host memory and back in with each engine, through pairs from the
    block manager.  `shuffled`: device blocks from a shuffled free list (one
    runtime copy per block and pool); `contiguous`: ascending device blocks
    (one runtime copy per pool on the way out; swap-in takes the freed blocks
    back last retired first, so its runs are single blocks again).  Times are
    HIP events on the stream around `reps` back-to-back calls.  recompute_floor_us prices the other recovery option
    for the same layer from what the head layout fixes: the Q/K/V/O
    projections (2 * hidden * (2 * hidden + 2 * kv_width) FLOPs per token)
    plus causal attention over the prompt, at the dense bf16 MFMA peak, no
    MLP: any real layer recomputes slower than this."""
    B, hkv, d, hq = 16, 8, 128, 32
    hidden, kv_width = hq * d, hkv * d
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    max_blocks = -(-max(lengths) // B)
    nb = 2 * max_blocks
    kp = torch.randn((nb, B, hkv, d), device=dev, dtype=torch.float32).to(torch.bfloat16)
    vp = torch.randn((nb, B, hkv, d), device=dev, dtype=torch.float32).to(torch.bfloat16)
    pool = pk.KvPool(kp, vp)
    hk = torch.empty((max_blocks, B, hkv, d), dtype=torch.bfloat16).pin_memory()
    hv = torch.empty((max_blocks, B, hkv, d), dtype=torch.bfloat16).pin_memory()
    host = pk.HostKvPool(hk, hv)
    engines = {"kernel": pk.PA_SWAP_ENGINE_KERNEL, "memcpy": pk.PA_SWAP_ENGINE_MEMCPY}

    def timed(pairs, direction, engine):
        for _ in range(2):
            pk.swap_blocks(pool, host, pairs, direction, engine, stream)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(reps):
            pk.swap_blocks(pool, host, pairs, direction, engine, stream)
        end.record(stream)
        host_us = (time.perf_counter() - t0) * 1e6 / reps
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps * 1e3, host_us

    rows = []
    for L in lengths:
        blocks = -(-L // B)
        nbytes = 2 * blocks * B * hkv * d * 2
        row = {"context_len": L, "blocks": blocks, "bytes": nbytes}
        for layout, order in (("shuffled", np.random.default_rng(L).permutation(nb)), ("contiguous", None)):
            bm = pk.BlockManager(nb, B, order)
            bm.set_host_blocks(max_blocks)
            bm.append(0, L)
            out_pairs = bm.swap_out([0])
            in_pairs = bm.swap_in([0])
            for ename, eng in engines.items():
                if layout == "contiguous" and ename == "kernel":
                    continue
                us_out, h_out = timed(out_pairs, pk.PA_SWAP_OUT, eng)
                us_in, h_in = timed(in_pairs, pk.PA_SWAP_IN, eng)
                key = f"{ename}_{layout}"
                row[key] = {"out_us": round(us_out, 2), "in_us": round(us_in, 2),
                            "out_GBs": round(nbytes / us_out / 1e3, 2), "in_GBs": round(nbytes / us_in / 1e3, 2),
                            "host_call_us": round(max(h_out, h_in), 2)}
        flops = L * 2 * hidden * (2 * hidden + 2 * kv_width) + 2 * 2 * (L * (L + 1) // 2) * hq * d
        row["recompute_floor_us"] = round(flops / 2.5e15 * 1e6, 2)
        best_swap = min(row[k]["out_us"] + row[k]["in_us"] for k in ("kernel_shuffled", "memcpy_shuffled"))
        row["swap_round_trip_us"] = round(best_swap, 2)
        row["swap_us_per_token"] = round(best_swap / L, 4)
        rows.append(row)
    big = rows[-1]
    print(json.dumps({"metric": "swap_round_trip_GBs", "value": round(2 * big["bytes"] / big["swap_round_trip_us"] / 1e3, 2),
                      "unit": "GB/s", "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "swap one layer (8 KV heads, head_dim 128, block 16) of a sequence "
                                             "to pinned host memory and back", "reps": reps},
                      "sweep": rows}), flush=True)
    return 0


def e2e_loop(torch, pk, w, pools, q_d, new_k, new_v, out, steps: int, build_plan, native_step=None,
             plan_reuse: int = 0) -> dict:
    """A serving loop over the workload's batch, `steps` decode steps long.
    Each step the host appends one token to every sequence (block manager),
    writes table rows and lengths, builds the plan for the new lengths,
    stages all of it in pinned host memory and uploads it, then launches
    pa_copy_blocks (when the append made copy-on-write pairs) and the fused
    pa_decode.  Launches are asynchronous, so the host prepares step n + 1
    while the GPU runs step n; the wall time per step is the larger of the
    two.  Lengths grow by one per step, as in serving.

    native_step = (num_workgroups, schedule, first_blocks): the host work is
    one pa_bm_prepare_decode_step call into a pinned buffer and one upload;
    otherwise (cascade plans) the separate binding calls, staged and uploaded
    one array at a time.  plan_reuse: the block manager advances its last
    plan (pa_bm_set_plan_reuse) for up to that many steps between builds."""
    bm, S, B, R = w["bm"], w["S"], w["B"], len(pools)
    seqs = np.arange(S)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    maxw = int(w["tables"].shape[1]) + -(-(steps + 1) // B) + 1
    probe_plan = build_plan(w["lens"], w["tables"])
    plan_cap = 4 * probe_plan.info.bytes + (1 << 16)
    ws = torch.empty(max(4 * pk.decode_workspace_bytes(probe_plan, w["hq"], w["d"]), 1 << 20) // 4,
                     dtype=torch.float32, device=dev)
    stage_done = [torch.cuda.Event() for _ in range(2)]
    if native_step is not None:
        nwg, sched, first = native_step
        bm.set_plan_reuse(plan_reuse)
        parts = {k: [] for k in ("wait", "prepare", "upload", "launch")}
        cap = 256 * (-(-(16 * S + 4 * S * maxw + 4 * S + plan_cap) // 256) + 8)
        stage = [torch.empty(cap, dtype=torch.uint8).pin_memory() for _ in range(2)]
        for st_ in stage:
            st_.numpy()[:] = 0
        # One device buffer, uploaded on the launch stream: an upload on a
        # copy stream of its own with event waits both ways measured slower
        # (190 against 82 us per step at C3).
        dev_buf = torch.empty(cap, dtype=torch.uint8, device=dev)
        views = None
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for k in range(steps):
            t0 = time.perf_counter()
            j = k % 2
            if k >= 2:
                stage_done[j].synchronize()       # the upload of step k - 2 has read this buffer
            tw = time.perf_counter()
            lay, plan = bm.prepare_decode_step(seqs, maxw, w["hkv"], stage[j], nwg, sched, first)
            t1 = time.perf_counter()
            dev_buf[:lay.bytes].copy_(stage[j][:lay.bytes], non_blocking=True)
            stage_done[j].record(stream)
            if views is None:                     # offsets depend only on S and maxw
                views = (dev_buf[lay.tables_at:lay.tables_at + 4 * S * maxw].view(torch.int32).view(S, maxw),
                         dev_buf[lay.lens_at:lay.lens_at + 4 * S].view(torch.int32),
                         dev_buf[lay.plan_at:],
                         dev_buf[lay.cows_at:lay.cows_at + 8 * S].view(torch.int32).view(S, 2))
            tables_e, lens_e, plan_e, cows_e = views
            t2 = time.perf_counter()
            pool = pools[k % R]
            if lay.n_cows:
                pk.copy_blocks(pool, cows_e[:lay.n_cows], stream)
            pk.decode(pool, q_d, tables_e, lens_e, w["case"]["scale"], plan, plan_e, ws, out, stream,
                      new_key=new_k, new_value=new_v)
            t3 = time.perf_counter()
            for name, a, b in (("wait", t0, tw), ("prepare", tw, t1), ("upload", t1, t2), ("launch", t2, t3)):
                parts[name].append((b - a) * 1e6)
        torch.cuda.synchronize()
        wall_us = (time.perf_counter() - t_start) * 1e6 / steps
    else:
        tables_e = torch.empty((S, maxw), dtype=torch.int32, device=dev)
        lens_e = torch.empty(S, dtype=torch.int32, device=dev)
        plan_e = torch.empty(plan_cap, dtype=torch.uint8, device=dev)
        cows_e = torch.empty((S, 2), dtype=torch.int32, device=dev)
        stage = [dict(tables=torch.empty((S, maxw), dtype=torch.int32).pin_memory(),
                      lens=torch.empty(S, dtype=torch.int32).pin_memory(),
                      plan=torch.empty(plan_cap, dtype=torch.uint8).pin_memory(),
                      cows=torch.empty((S, 2), dtype=torch.int32).pin_memory()) for _ in range(2)]
        parts = {k: [] for k in ("append", "export", "plan", "stage_upload", "launch")}
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for k in range(steps):
            t0 = time.perf_counter()
            _, cows = bm.append_step(seqs)
            t1 = time.perf_counter()
            tables, lens = bm.export(seqs, maxw)
            t2 = time.perf_counter()
            plan = build_plan(lens, tables)
            t3 = time.perf_counter()
            j = k % 2
            if k >= 2:
                stage_done[j].synchronize()       # the uploads of step k - 2 have read this staging set
            st = stage[j]
            st["tables"].numpy()[:] = tables
            st["lens"].numpy()[:] = lens
            nb = plan.info.bytes
            st["plan"].numpy()[:nb] = plan.blob
            tables_e.copy_(st["tables"], non_blocking=True)
            lens_e.copy_(st["lens"], non_blocking=True)
            plan_e[:nb].copy_(st["plan"][:nb], non_blocking=True)
            n_cow = len(cows)
            if n_cow:
                st["cows"].numpy()[:n_cow] = cows
                cows_e[:n_cow].copy_(st["cows"][:n_cow], non_blocking=True)
            stage_done[j].record(stream)
            t4 = time.perf_counter()
            pool = pools[k % R]
            if n_cow:
                pk.copy_blocks(pool, cows_e[:n_cow], stream)
            pk.decode(pool, q_d, tables_e, lens_e, w["case"]["scale"], plan, plan_e, ws, out, stream,
                      new_key=new_k, new_value=new_v)
            t5 = time.perf_counter()
            for name, a, b in (("append", t0, t1), ("export", t1, t2), ("plan", t2, t3), ("stage_upload", t3, t4),
                               ("launch", t4, t5)):
                parts[name].append((b - a) * 1e6)
        torch.cuda.synchronize()
        wall_us = (time.perf_counter() - t_start) * 1e6 / steps
    host = {name: round(float(np.median(v)), 2) for name, v in parts.items()}
    host_total = round(float(np.median([sum(x) for x in zip(*parts.values())])), 2)
    return {"steps": steps, "us_per_step": round(wall_us, 2), "decode_tokens_per_s": round(S / (wall_us * 1e-6), 1),
            "host_path": (f"pa_bm_prepare_decode_step, one upload; the plan built every {plan_reuse + 1} steps and "
                          "advanced (pa_decode_plan_advance) in between" if plan_reuse else
                          "pa_bm_prepare_decode_step, one upload") if native_step is not None else
                         "separate binding calls, one upload per array",
            "host_us_median": host, "host_total_us_median": host_total,
            "note": "wall time per step of the whole serving loop (host block manager, plan, uploads and the GPU "
                    "launches of one attention layer), lengths growing by one per step; a model's other layers "
                    "reuse the step's plan and tables"}


def length_sweep(torch, pk, lengths=(16, 32, 64, 128, 200, 256, 400, 640), reps: int = 100) -> int:
    """Attention launch time against KV bytes for batches of 256 sequences of
    one length each (c3 heads: 32 q / 8 KV, head_dim 128, block 16, shuffled
    blocks): one job per workgroup and no merge, so time = fixed cost + bytes
    / streaming rate.  The fit over lengths >= 64 separates the two."""
    S, hq, hkv, d, B = 256, 32, 8, 128, 16
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    rows = []
    for L in lengths:
        lens = np.full(S, L, np.int32)
        nblk = -(-lens // B)
        nb = int(nblk.sum()) + S
        perm = np.random.default_rng(L).permutation(nb).astype(np.int32)
        maxb = int(nblk.max())
        tables = np.zeros((S, maxb), np.int32)
        off = 0
        for s in range(S):
            tables[s, :nblk[s]] = perm[off:off + nblk[s]]
            off += nblk[s]
        R = max(2, -(-2**30 // (2 * nb * B * hkv * d * 2)))
        pools = [pk.KvPool(torch.randn((nb, B, hkv, d), device=dev).to(torch.bfloat16),
                           torch.randn((nb, B, hkv, d), device=dev).to(torch.bfloat16)) for _ in range(R)]
        plan = pk.decode_plan(lens, hkv).set_first_blocks(tables, B)
        plan_d = plan.to_device(dev)
        ws = torch.empty(max(pk.decode_workspace_bytes(plan, hq, d), 256) // 4, device=dev)
        q = torch.randn((S, hq, d), device=dev).to(torch.bfloat16)
        out = torch.empty((S, hq, d), device=dev)
        td, ld = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
        for i in range(10):
            pk.decode(pools[i % R], q, td, ld, 0.088, plan, plan_d, ws, out, stream, stage="attention")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            pk.decode(pools[i % R], q, td, ld, 0.088, plan, plan_d, ws, out, stream, stage="attention")
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        nbytes = int(lens.sum()) * hkv * d * 2 * 2
        rows.append({"context_len": L, "us": round(us, 2), "bytes": nbytes, "GBs": round(nbytes / us / 1e3, 1),
                     "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
        del pools
    x = np.array([r["bytes"] for r in rows if r["context_len"] >= 64], float)
    y = np.array([r["us"] for r in rows if r["context_len"] >= 64], float)
    slope, fixed = np.polyfit(x, y, 1)
    print(json.dumps({"metric": "attention launch time against KV bytes", "fixed_us": round(float(fixed), 2),
                      "streaming_GBs": round(float(1e3 / (slope * 1e9) * 1e3), 1),
                      "config": {"workload": "256 sequences of one length, 32 q / 8 KV heads, head_dim 128, "
                                             "block 16, bf16", "reps": reps}, "sweep": rows}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first: an idle GPU runs its first milliseconds of work slower")
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--block-size", type=int, default=None, choices=(1, 2, 4, 8, 16, 32),
                    help="block size (default: the workload's; c5, c6: 16)")
    ap.add_argument("--workgroups", type=int, default=None, help="persistent workgroups (default: fill the GPU)")
    ap.add_argument("--piece", type=int, default=0, help="longest job piece in 16-token tiles (0: auto)")
    ap.add_argument("--schedule", default="auto", choices=("auto", "chunks", "lpt"),
                    help="host schedule (auto: the cheaper of the two by the planner's cost)")
    ap.add_argument("--replicas", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true", help="time only pa_decode launches (profiling aid)")
    ap.add_argument("--graph", action="store_true", help="replay each step as a captured HIP graph")
    ap.add_argument("--no-cascade", action="store_true",
                    help="c5, c6: plan every sequence separately instead of reading shared prefixes once per group")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="profiling aid: run a plain device-to-device copy of BYTES (the reference whose "
                         "counter readings calibrate the traffic figures) and exit")
    ap.add_argument("--no-first-blocks", action="store_true",
                    help="leave the jobs' first-tile table entries out of the plan (the first tile loads then "
                         "wait for a table load)")
    ap.add_argument("--length-sweep", action="store_true",
                    help="time the attention launch for uniform batches of 16..640 tokens and fit fixed cost "
                         "and streaming rate, then exit")
    ap.add_argument("--read-probe", action="store_true",
                    help="time a plain streaming read (pa_probe_read) at 16 MB .. 1 GiB, fit fixed cost and "
                         "streaming rate, and exit")
    ap.add_argument("--plan-reuse", type=int, default=15,
                    help="end-to-end loop: steps a plan is advanced (pa_decode_plan_advance) before it is rebuilt")
    ap.add_argument("--e2e-steps", type=int, default=32,
                    help="steps of the end-to-end serving loop timed last (host append, export, plan and upload "
                         "of every step overlapped with the GPU step before it); 0 skips it")
    ap.add_argument("--swap-sweep", action="store_true",
                    help="measure swapping a sequence out to pinned host memory and back at several context "
                         "lengths (both engines) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path is single-GPU; see the sharding notes in the design document)", file=sys.stderr)
        return 2

    import torch
    if args.copy_probe:
        return copy_probe(torch, args.copy_probe)
    import paged_kv_cache_115_amd as pk
    if args.swap_sweep:
        torch.cuda.set_device(0)
        return swap_sweep(torch, pk, [256, 1024, 4096, 16384, 32768])
    if args.length_sweep:
        torch.cuda.set_device(0)
        return length_sweep(torch, pk)
    if args.read_probe:
        torch.cuda.set_device(0)
        return read_probe_sweep(torch, pk)

    torch.cuda.set_device(0)
    if args.config == "c5":
        w = prefix_workload(pk, args.block_size or 16)
    elif args.config == "c6":
        w = prefix_cache_workload(pk, args.block_size or 16)
    else:
        w = decode_workload(pk, args.config, args.block_size)
    name, case = w["name"], w["case"]
    S, hq, hkv, d, B, nb = w["S"], w["hq"], w["hkv"], w["d"], w["B"], w["nb"]
    tables, lens, slots, cows = w["tables"], w["lens"], w["slots"], w["cows"]
    host_append_us = w["host_append_us"]
    workgroups = args.workgroups or pk.default_workgroups()
    cascade = "prefix_group" in w and not args.no_cascade
    def build_plan():
        if cascade:
            p = pk.decode_plan_prefix(lens, hkv, hq, w["prefix_group"], w["prefix_tokens"], workgroups, args.piece,
                                      block_size=B)
        else:
            sched = {"auto": pk.SCHEDULE_AUTO, "chunks": pk.SCHEDULE_CHUNKS, "lpt": pk.SCHEDULE_LPT}[args.schedule]
            p = pk.decode_plan(lens, hkv, workgroups, args.piece, shared_kv=w["shared_kv"], schedule=sched,
                               block_size=B)
        if not args.no_first_blocks:
            p.set_first_blocks(tables, B)
        return p

    # Host plan time: median of warm builds through the Python binding (a
    # serving loop builds one per step; the first call also sizes buffers).
    plan_times = []
    for _ in range(21):
        t0 = time.perf_counter()
        plan = build_plan()
        plan_times.append((time.perf_counter() - t0) * 1e6)
    host_plan_us = float(np.median(plan_times[1:]))

    dev = torch.device("cuda", 0)
    f32 = case.get("cfg", {}).get("dtype") == "f32"
    kv_dtype, e = (torch.float32, 4) if f32 else (torch.bfloat16, 2)
    tables_d = torch.from_numpy(tables).to(dev)
    lens_d = torch.from_numpy(lens).to(dev)
    plan_d = plan.to_device(dev)
    slots_d = torch.from_numpy(slots).to(dev)
    cows_d = torch.from_numpy(np.ascontiguousarray(cows, dtype=np.int32)).to(dev)
    ws_bytes = pk.decode_workspace_bytes(plan, hq, d)
    ws = torch.empty(max(ws_bytes, 256) // 4, dtype=torch.float32, device=dev)
    q_d = (torch.from_numpy(case["q"]) if f32 else torch.from_numpy(case["q"].view(np.int16)).view(torch.bfloat16)).to(dev)

    pool_bytes = 2 * nb * B * hkv * d * e
    R = args.replicas or max(2, math.ceil(2**30 / pool_bytes))
    # All replicas' K pools and the new K rows in one allocation, and the same
    # for V, so that each pool and the new rows share one 4 GiB window (the
    # fused append then reads every tile with buffer loads; the mode is
    # reported in the config).
    pool_elems, new_elems = nb * B * hkv * d, S * hkv * d
    k_slab = torch.empty(R * pool_elems + new_elems, dtype=kv_dtype, device=dev)
    v_slab = torch.empty(R * pool_elems + new_elems, dtype=kv_dtype, device=dev)
    pools = []
    for r in range(R):
        g = torch.Generator(device=dev)
        g.manual_seed(w["seed"] + 1000 * r)
        kp = k_slab[r * pool_elems:(r + 1) * pool_elems].view(nb, B, hkv, d)
        vp = v_slab[r * pool_elems:(r + 1) * pool_elems].view(nb, B, hkv, d)
        kp.copy_(torch.randn((nb, B, hkv, d), generator=g, device=dev, dtype=torch.float32))
        vp.copy_(torch.randn((nb, B, hkv, d), generator=g, device=dev, dtype=torch.float32))
        pools.append(pk.KvPool(kp, vp))
    g = torch.Generator(device=dev)
    g.manual_seed(w["seed"] + 7)
    new_k = k_slab[R * pool_elems:].view(S, hkv, d)
    new_v = v_slab[R * pool_elems:].view(S, hkv, d)
    new_k.copy_(torch.randn((S, hkv, d), generator=g, device=dev))
    new_v.copy_(torch.randn((S, hkv, d), generator=g, device=dev))
    out = torch.empty((S, hq, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(r: int, st=None):
        st = st or stream
        pool = pools[r]
        if not args.decode_only:
            pk.copy_blocks(pool, cows_d, st)
            pk.reshape_and_cache(pool, new_k, new_v, slots_d, st)
        pk.decode(pool, q_d, tables_d, lens_d, case["scale"], plan, plan_d, ws, out, st)

    def step_fused(r: int, st=None):
        # The step: the append fused into pa_decode, which stores every
        # sequence's token L - 1 from new_k/new_v into its slot.
        st = st or stream
        pool = pools[r]
        if not args.decode_only:
            pk.copy_blocks(pool, cows_d, st)
        pk.decode(pool, q_d, tables_d, lens_d, case["scale"], plan, plan_d, ws, out, st,
                  new_key=new_k, new_value=new_v)

    def attention(r: int):
        # The step's attention launch (append fused).
        pk.decode(pools[r], q_d, tables_d, lens_d, case["scale"], plan, plan_d, ws, out, stream, stage="attention",
                  new_key=new_k, new_value=new_v)

    def attention_unfused(r: int):
        pk.decode(pools[r], q_d, tables_d, lens_d, case["scale"], plan, plan_d, ws, out, stream, stage="attention")

    def decode_call(r: int):
        pk.decode(pools[r], q_d, tables_d, lens_d, case["scale"], plan, plan_d, ws, out, stream,
                  new_key=new_k, new_value=new_v)

    def timed(fn, n: int) -> float:
        """Milliseconds per call of n back-to-back calls, from HIP events
        recorded on the launch stream, bracketed by synchronisation."""
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(n):
            fn(k % R)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    def timed_blocks(fn, blocks: int = 40, per: int = 10) -> dict:
        """Distribution of per-call times: `blocks` blocks of `per` back-to-back
        calls, an event between blocks (an event between every two calls would
        cost more than the spread it measures); microseconds per call of
        each block, summarised by percentiles."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        k = 0
        for b in range(blocks):
            for _ in range(per):
                fn(k % R)
                k += 1
            ev[b + 1].record(stream)
        torch.cuda.synchronize()
        us = [ev[b].elapsed_time(ev[b + 1]) / per * 1e3 for b in range(blocks)]
        return dict(percentiles(us), blocks=blocks, calls_per_block=per)

    for k in range(args.warmup):
        step_fused(k % R)
    torch.cuda.synchronize()

    # The timed region: K whole steps.
    ms_per_step = timed(step_fused, args.steps)
    if args.graph:
        # One step per pool replica captured as a HIP graph, replayed in turn.
        cap = torch.cuda.Stream()
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step_fused(r, cap)
            graphs.append(g)
        for k in range(args.warmup):
            graphs[k % R].replay()
        torch.cuda.synchronize()
        ms_per_step = timed(lambda r: graphs[r].replay(), args.steps)
    # The same step as three calls, after its own warm-up.
    for k in range(args.warmup):
        step(k % R)
    ms_per_step_eager = timed(step, args.steps)
    # The dominant kernel alone: K attention launches back to back (same
    # inputs, rotating pool replicas); the same without the fused append; K
    # whole pa_decode calls.
    attention_us = timed(attention, args.steps) * 1e3
    attention_unfused_us = timed(attention_unfused, args.steps) * 1e3
    decode_us = timed(decode_call, args.steps) * 1e3
    # Spread of the step and of its attention launch (separate regions, after
    # the timed ones).
    step_stats = timed_blocks(step_fused)
    attention_stats = timed_blocks(attention)
    pk.decode(pools[0], q_d, tables_d, lens_d, case["scale"], plan, plan_d, ws, out, stream)   # leave a complete result
    torch.cuda.synchronize()

    # Algorithmic KV bytes: every distinct (block, slot) the step reads, K and
    # V of every KV head, once (equal to the logical bytes unless sequences
    # share blocks).
    kv_bytes = w["unique_tokens"] * hkv * d * 2 * e
    logical_kv_bytes = int(lens.astype(np.int64).sum()) * hkv * d * 2 * e
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (attention_us * 1e-6) / 1e9
    schedule = [int(workgroups), int(args.piece)]
    result = {
        "metric": "paged decode attention KV-read GB/s (% of HBM peak) and decode tokens/s, 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_eager": round(ms_per_step_eager, 5),
        "graph": bool(args.graph),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if f32 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{name}: {w['desc']}", "num_seqs": S, "num_q_heads": hq,
                   "num_kv_heads": hkv, "head_dim": d, "block_size": B,
                   "total_context_tokens": int(lens.sum()), "max_context": int(lens.max()),
                   "workgroups": int(workgroups), "max_piece_tiles": int(args.piece),
                   "jobs": int(plan.num_jobs), "merges": int(plan.num_merges), "records": int(plan.num_records),
                   "pool_replicas": R, "decode_only": bool(args.decode_only), "shared_kv": bool(w["shared_kv"]),
                   "schedule": ["chunks", "largest pieces first"][plan.schedule],
                   "cascade_prefix_groups": int(plan.num_groups) if cascade else 0,
                   "first_tile_entries": not args.no_first_blocks,
                   "kv_loads": "cached" if plan.info.flags & pk.PA_DECODE_SHARED_KV else "streamed",
                   "fused_loads": pk.FUSED_LOADS[pk.decode_fused_loads(pools[0], new_k, new_v, plan, hq)]},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(S / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "logical_kv_bytes_per_step": logical_kv_bytes,
        "logical_kv_GBs": round(logical_kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "copy_blocks_per_step": int(len(cows)),
        # block-size trade-off: slots reserved by the tables against live tokens (tail waste)
        "reserved_slots": int(sum(-(-int(L) // B) * B for L in lens)),
        "tail_waste_frac": round(1 - int(lens.sum()) / max(1, sum(-(-int(L) // B) * B for L in lens)), 5),
        "table_entries_per_seq": round(float(np.mean([-(-int(L) // B) for L in lens])), 2),
        "us_per_output_token": round(ms_per_step * 1e3 / S, 5),
        "step_us_stats": step_stats,
        "decode_call_us": round(decode_us, 3),
        "attention_launch_us": round(attention_us, 3),
        "attention_launch_us_stats": attention_stats,
        "attention_launch_unfused_us": round(attention_unfused_us, 3),
        "unfused_frac": round(kv_bytes / (attention_unfused_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "host_append_us": round(host_append_us, 2),
        "host_plan_us": round(host_plan_us, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name, schedule),
                     "kernel": ("decode_f32_kernel" if f32 else "decode_bf16_kernel") +
                               " (the attention launch of pa_decode, append fused)",
                     "bytes_per_launch": kv_bytes},
    }
    if "prefix_cache" in w:
        result["prefix_cache"] = w["prefix_cache"]
    # The achievable read rate for the same bytes: a plain streaming read of
    # that many bytes on the same grid size.
    probe = read_probe(torch, pk, kv_bytes - kv_bytes % 16)
    result["read_probe"] = dict(probe, attention_vs_probe=round(probe["us"] / attention_us, 4))
    if not args.decode_only:
        result["copy_blocks_probe"] = copy_blocks_probe(torch, pk, B, hkv, d)
    if args.e2e_steps > 0:
        # Last: it advances the block manager's sequences.
        def plan_for(lens_h, tables_h):
            if cascade:
                grp, tok = w["bm"].prefix_groups(np.arange(S))
                p = pk.decode_plan_prefix(lens_h, hkv, hq, grp, tok, workgroups, args.piece, block_size=B)
            else:
                sched = {"auto": pk.SCHEDULE_AUTO, "chunks": pk.SCHEDULE_CHUNKS, "lpt": pk.SCHEDULE_LPT}[args.schedule]
                p = pk.decode_plan(lens_h, hkv, workgroups, args.piece, shared_kv=w["shared_kv"], schedule=sched,
                                   block_size=B)
            if not args.no_first_blocks:
                p.set_first_blocks(tables_h, B)
            return p
        native = None if cascade else (workgroups, plan.schedule if args.schedule == "auto" else
                                       {"chunks": pk.SCHEDULE_CHUNKS, "lpt": pk.SCHEDULE_LPT}[args.schedule],
                                       not args.no_first_blocks)
        e2e = e2e_loop(torch, pk, w, pools, q_d, new_k, new_v, out, args.e2e_steps, plan_for, native,
                       args.plan_reuse)
        if native is not None:
            e2e["schedule"] = ["chunks", "largest pieces first"][native[1]] + \
                " (the automatic choice for the batch at the first step, kept)"
        result["e2e"] = e2e
        result["decode_tokens_per_s_gpu_only"] = result["decode_tokens_per_s"]
        result["decode_tokens_per_s"] = e2e["decode_tokens_per_s"]
    if not args.no_cpu_baseline:
        if f32:
            k_host, v_host = pools[0].k.cpu().numpy(), pools[0].v.cpu().numpy()
        else:
            k_host = pools[0].k.cpu().view(torch.int16).numpy().view(np.uint16)
            v_host = pools[0].v.cpu().view(torch.int16).numpy().view(np.uint16)
        result["cpu_baseline"] = cpu_baseline(case, hkv * d * 2 * e, k_host, v_host, tables, lens, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
