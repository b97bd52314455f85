"""Seeded synthetic inputs for paged decode attention.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests.  It holds input synthesis only: length draws, the order in which the
free list hands out physical blocks, token keys/values, queries and pool fill
patterns.  It computes no part of the method itself: no block table, no slot
address, no attention.  Block tables and slots are produced on each side by its
own block manager from the free-list order drawn here.

Workloads follow the pages' descriptions of typical traffic:
  * replies averaging about 200 tokens with a heavy tail (mercemay.com, "Paged
    KV Cache Allocation and the Block Table", section "The arithmetic is stark"
    paragraph and "Three ways contiguous reservation loses memory");
  * a 4096-token context limit (aicassindra.com, "tm_paged_attention_deep",
    "Why contiguous KV allocation bleeds memory");
  * a 2,000-token shared prompt sampled n=4 times (llminference.xinbetween.com
    S06 "PagedAttention", "Copy-on-write, for free");
  * block size 16 as the common default (same page, "Choosing the block size").

Draw order for one case: lengths, then the free-list order, then keys and
values (standard normal, float32, rounded to nearest-even bfloat16 for bf16
cases), then queries.
"""
from __future__ import annotations

import math
import os

import numpy as np

# Named workloads.  The "small" variants keep the structure of the full ones
# (head counts, head_dim, block size, length mix) at sizes a float64 oracle
# finishes in seconds while still spanning several 16-token tiles, several
# context partitions and a ragged final block.
CONFIGS: dict[str, dict] = {
    # 4 sequences, fp32, one appended token each.
    "c1": dict(seed=1, num_seqs=4, num_q_heads=4, num_kv_heads=4, head_dim=64,
               block_size=16, dtype="f32", lengths=("fixed", [1, 17, 33, 100]),
               pool_blocks=64),
    # MHA, batch 64, lengths uniform on [1, 2048].
    "c2": dict(seed=2, num_seqs=64, num_q_heads=32, num_kv_heads=32, head_dim=128,
               block_size=16, dtype="bf16", lengths=("uniform", 1, 2048)),
    # GQA group 4, batch 256, lognormal lengths with mean 200, capped at 4096.
    "c3": dict(seed=3, num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
               block_size=16, dtype="bf16",
               lengths=("lognormal", math.log(200.0) - 0.5, 1.0, 1, 4096)),
    # The batch-256 GQA batch with an fp32 pool (the same lengths as c3).
    "c3f": dict(seed=3, num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, dtype="f32",
                lengths=("lognormal", math.log(200.0) - 0.5, 1.0, 1, 4096)),
    # Long context GQA group 8, batch 16, lengths uniform on [16384, 32768].
    "c4": dict(seed=4, num_seqs=16, num_q_heads=64, num_kv_heads=8, head_dim=128,
               block_size=16, dtype="bf16", lengths=("uniform", 16384, 32768),
               partition_size=512),
    # --- reduced-size variants used where the oracle must see every output ---
    "c2s": dict(seed=12, num_seqs=8, num_q_heads=32, num_kv_heads=32, head_dim=128,
                block_size=16, dtype="bf16", lengths=("uniform", 1, 300)),
    "c3s": dict(seed=13, num_seqs=24, num_q_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, dtype="bf16",
                lengths=("lognormal", math.log(200.0) - 0.5, 1.0, 1, 700)),
    "c4s": dict(seed=14, num_seqs=3, num_q_heads=64, num_kv_heads=8, head_dim=128,
                block_size=16, dtype="bf16", lengths=("uniform", 1500, 3000),
                partition_size=512),
}

# Prefix sharing with copy-on-write: prompts x samples sharing a prefix.
PREFIX_CONFIGS: dict[str, dict] = {
    "c5": dict(seed=5, num_prompts=32, samples=4, prefix_len=2000, tail=(1, 512),
               num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
               block_sizes=(8, 16, 32)),
    "c5s": dict(seed=15, num_prompts=3, samples=4, prefix_len=100, tail=(1, 40),
                num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                block_sizes=(8, 16, 32)),
    # More samples per prompt than one group of a shared read holds (c6's
    # shape at oracle size: each prompt's prefix is shared by several groups).
    "c5w": dict(seed=35, num_prompts=3, samples=14, prefix_len=300, tail=(1, 40),
                num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                block_sizes=(8, 16, 32)),
}

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); finite input only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


_CHUNK = 1 << 22   # elements per independently seeded chunk of a normal draw


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """Standard normal float32 values (rounded to bfloat16 for "bf16").

    The case generator draws one 64-bit seed; the array is filled in chunks of
    _CHUNK elements, chunk i from its own generator spawned as child i of that
    seed.  Chunks are independent, so they are filled in parallel threads and
    the result does not depend on the thread count."""
    n = int(np.prod(shape))
    seed = int(rng.integers(0, 2**63))
    nchunks = max(1, -(-n // _CHUNK))
    children = np.random.SeedSequence(seed).spawn(nchunks)
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)

    def fill(i: int) -> None:
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = np.random.default_rng(children[i]).standard_normal(size=hi - lo, dtype=np.float32)
        out[lo:hi] = x if dtype == "f32" else f32_to_bf16_bits(x)

    if nchunks == 1:
        fill(0)
    else:
        from concurrent.futures import ThreadPoolExecutor
        workers = min(nchunks, max(1, min(16, len(os.sched_getaffinity(0)))))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(fill, range(nchunks)))
    return out.reshape(shape)


def element_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) as the float32 value handed to both sides."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def draw_lengths(cfg: dict, rng: np.random.Generator) -> np.ndarray:
    kind = cfg["lengths"][0]
    n = cfg["num_seqs"]
    if kind == "fixed":
        out = np.asarray(cfg["lengths"][1], dtype=np.int64)
    elif kind == "uniform":
        lo, hi = cfg["lengths"][1], cfg["lengths"][2]
        out = rng.integers(lo, hi + 1, size=n)
    elif kind == "lognormal":
        mu, sigma, lo, hi = cfg["lengths"][1:]
        out = np.clip(np.rint(rng.lognormal(mu, sigma, size=n)), lo, hi)
    else:
        raise ValueError(kind)
    return out.astype(np.int32)


def pool_blocks_for(lengths: np.ndarray, block_size: int, slack: float = 1.25) -> int:
    """Pool size rule: `slack` times the live tokens in blocks, plus one spare
    block per sequence for its partly filled tail block."""
    return int(slack * (int(lengths.sum()) // block_size + len(lengths))) + 1


def decode_case(name: str, seed: int | None = None) -> dict:
    """One decode step's inputs for a named workload.

    Keys of the result:
      cfg, lengths[S] (tokens attended, counting this step's appended token),
      free_order[NB] (order in which physical blocks leave the free list),
      keys/values [sum(L), Hkv, D] in logical order, sequence after sequence
        (token t of sequence s at row offsets[s] + t; the last row of each
        sequence is this step's appended token),
      offsets[S+1], q[S, Hq, D], scale, num_blocks.
    fp32 arrays are float32; bf16 arrays are uint16 bit patterns.
    """
    cfg = dict(CONFIGS[name])
    rng = np.random.default_rng(cfg["seed"] if seed is None else seed)
    lengths = draw_lengths(cfg, rng)
    nb = cfg.get("pool_blocks") or pool_blocks_for(lengths, cfg["block_size"])
    free_order = rng.permutation(nb).astype(np.int32)
    total = int(lengths.sum())
    hkv, d, dt = cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    keys = _normal(rng, (total, hkv, d), dt)
    values = _normal(rng, (total, hkv, d), dt)
    q = _normal(rng, (len(lengths), cfg["num_q_heads"], d), dt)
    offsets = np.zeros(len(lengths) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lengths)
    return dict(cfg=cfg, name=name, lengths=lengths, free_order=free_order,
                keys=keys, values=values, offsets=offsets, q=q,
                scale=default_scale(d), num_blocks=nb)


def prefix_case(name: str, block_size: int, seed: int | None = None) -> dict:
    """Prompts sampled `samples` times: a shared prefix plus a private tail each.

    Keys: cfg, prefix_keys/prefix_values [P, prefix_len, Hkv, D],
    tail_lengths[P*n] (tail tokens per sample, sample j of prompt p at p*n+j),
    tail_keys/tail_values [sum(tail), Hkv, D], tail_offsets[P*n+1],
    q[P*n, Hq, D], free_order[NB], scale, num_blocks.
    """
    cfg = dict(PREFIX_CONFIGS[name])
    rng = np.random.default_rng(cfg["seed"] + block_size if seed is None else seed)
    p, n, pre = cfg["num_prompts"], cfg["samples"], cfg["prefix_len"]
    lo, hi = cfg["tail"]
    tails = rng.integers(lo, hi + 1, size=p * n).astype(np.int32)
    shared_tokens = p * pre + int(tails.sum())
    nb = int(1.25 * (shared_tokens // block_size)) + 2 * p * n + 1
    free_order = rng.permutation(nb).astype(np.int32)
    hkv, d, dt = cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    prefix_keys = _normal(rng, (p, pre, hkv, d), dt)
    prefix_values = _normal(rng, (p, pre, hkv, d), dt)
    tail_keys = _normal(rng, (int(tails.sum()), hkv, d), dt)
    tail_values = _normal(rng, (int(tails.sum()), hkv, d), dt)
    q = _normal(rng, (p * n, cfg["num_q_heads"], d), dt)
    tail_offsets = np.zeros(p * n + 1, dtype=np.int64)
    tail_offsets[1:] = np.cumsum(tails)
    return dict(cfg=cfg, name=name, block_size=block_size, tail_lengths=tails,
                prefix_keys=prefix_keys, prefix_values=prefix_values,
                tail_keys=tail_keys, tail_values=tail_values,
                tail_offsets=tail_offsets, q=q, free_order=free_order,
                scale=default_scale(d), num_blocks=nb)


# Preemption: a pool too small for the batch's growth, so that decode steps run
# the allocator dry and sequences are swapped to host memory and back
# (mercemay.com "Paged KV Cache Allocation and the Block Table", "Three ways
# contiguous reservation loses memory"; llminference.xinbetween.com S06, third
# exercise).  Prompt lengths follow the c3 mix, capped low; one prompt is
# sampled three times (fork) so that shared blocks are swapped too.
PREEMPT_CONFIGS: dict[str, dict] = {
    "p1s": dict(seed=21, num_seqs=8, samples=3, prompt=(20, 200), steps=64, block_size=16,
                num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                pool_slack=1.15, host_blocks=96, retire_at=(24, 40), group_out_at=10),
    "p1f": dict(seed=22, num_seqs=6, samples=2, prompt=(10, 90), steps=48, block_size=8,
                num_q_heads=8, num_kv_heads=4, head_dim=64, dtype="f32",
                pool_slack=1.10, host_blocks=80, retire_at=(20, 30), group_out_at=16),
}


def preempt_case(name: str, seed: int | None = None) -> dict:
    """Inputs of a decode run that outgrows its pool.

    Keys: cfg, prompts[S] (prompt tokens per sequence), free_order[NB],
    rows_k/rows_v [R, Hkv, D] (token rows in the order they are appended,
    whichever sequence appends them; R bounds every run), q[S + samples - 1,
    Hq, D] (one query per sequence that can be alive at the end), scale,
    num_blocks, host_blocks."""
    cfg = dict(PREEMPT_CONFIGS[name])
    rng = np.random.default_rng(cfg["seed"] if seed is None else seed)
    lo, hi = cfg["prompt"]
    s, b = cfg["num_seqs"], cfg["block_size"]
    prompts = rng.integers(lo, hi + 1, size=s).astype(np.int32)
    nb = int(cfg["pool_slack"] * sum(-(-int(p) // b) for p in prompts)) + 1
    free_order = rng.permutation(nb).astype(np.int32)
    hkv, d, dt = cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    alive = s + cfg["samples"] - 1
    rows = int(prompts.sum()) + cfg["steps"] * alive
    rows_k = _normal(rng, (rows, hkv, d), dt)
    rows_v = _normal(rng, (rows, hkv, d), dt)
    q = _normal(rng, (alive, cfg["num_q_heads"], d), dt)
    return dict(cfg=cfg, name=name, prompts=prompts, free_order=free_order, rows_k=rows_k,
                rows_v=rows_v, q=q, scale=default_scale(d), num_blocks=nb,
                host_blocks=cfg["host_blocks"])


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
    return x ^ (x >> 31)


def token_rows(tokens, hkv: int, d: int, dtype: str, salt: int = 0, start: int = 0):
    """Stand-in for a model's keys and values of a token sequence: row t is
    drawn from a generator seeded by the whole prefix tokens[:t+1] (a rolling
    64-bit state), so two sequences get bit-identical rows exactly where
    their prefixes agree.  Returns (keys, values) [n - start, Hkv, D] for
    positions start .. n - 1."""
    n = len(tokens)
    k = np.empty((n - start, hkv, d), dtype=np.float32 if dtype == "f32" else np.uint16)
    v = np.empty_like(k)
    state = _splitmix64(salt)
    for t, tok in enumerate(tokens):
        state = _splitmix64(state ^ (int(tok) & 0xFFFFFFFF))
        if t < start:
            continue
        x = np.random.default_rng(state).standard_normal(size=(2, hkv, d), dtype=np.float32)
        if dtype != "f32":
            x = f32_to_bf16_bits(x)
        k[t - start], v[t - start] = x[0], x[1]
    return k, v


# Prefix caching across requests: requests that open with one of a few
# system prompts (the pages' example: the same 2,000-token system prompt sent
# thousands of times an hour; llminference.xinbetween.com S06, "What's next"
# and "Unshareable duplicates"), each followed by a private user turn.
PREFIX_CACHE_CONFIGS: dict[str, dict] = {
    "h1s": dict(seed=31, requests=12, system_prompts=2, system_len=(40, 90), user=(1, 50), vocab=50,
                block_size=16, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16"),
    "h1f": dict(seed=32, requests=10, system_prompts=3, system_len=(8, 40), user=(1, 20), vocab=7,
                block_size=8, num_q_heads=8, num_kv_heads=4, head_dim=64, dtype="f32"),
    # Full size: 256 requests over four 2,000-token system prompts, user turns
    # averaging 200 tokens, the c3 head layout.
    "c6": dict(seed=6, requests=256, system_prompts=4, system_len=(2000, 2000), user=(1, 400), vocab=32000,
               block_size=16, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16"),
}


def prefix_cache_case(name: str, seed: int | None = None) -> dict:
    """Token-id prompts of a request stream.  Keys: cfg, prompts (list of int32
    arrays, one per request in arrival order), system (which system prompt each
    request opens with), q[requests, Hq, D], scale, num_blocks (room for every
    prompt privately, plus one block per request)."""
    cfg = dict(PREFIX_CACHE_CONFIGS[name])
    rng = np.random.default_rng(cfg["seed"] if seed is None else seed)
    lo, hi = cfg["system_len"]
    systems = [rng.integers(0, cfg["vocab"], size=int(rng.integers(lo, hi + 1))).astype(np.int32)
               for _ in range(cfg["system_prompts"])]
    which = rng.integers(0, cfg["system_prompts"], size=cfg["requests"])
    ulo, uhi = cfg["user"]
    prompts = [np.concatenate([systems[w], rng.integers(0, cfg["vocab"], size=int(rng.integers(ulo, uhi + 1)))
                               .astype(np.int32)]) for w in which]
    b = cfg["block_size"]
    nb = sum(-(-len(p) // b) for p in prompts) + cfg["requests"]
    q = _normal(rng, (cfg["requests"], cfg["num_q_heads"], cfg["head_dim"]), cfg["dtype"])
    return dict(cfg=cfg, name=name, prompts=prompts, system=which, q=q, scale=default_scale(cfg["head_dim"]),
                num_blocks=nb)


def byte_pattern(shape, dtype: str, seed: int) -> np.ndarray:
    """Seeded arbitrary bit patterns (any bits, NaNs included) for copy tests."""
    rng = np.random.default_rng(seed)
    if dtype == "f32":
        return rng.integers(0, 2**32, size=shape, dtype=np.uint32).view(np.float32)
    return rng.integers(0, 2**16, size=shape, dtype=np.uint16)


def nan_fill(shape, dtype: str) -> np.ndarray:
    """Pool fill marking never-written slots: every element is a quiet NaN."""
    if dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, BF16_NAN, dtype=np.uint16)
