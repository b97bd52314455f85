"""Float64 CPU oracle: decode attention through a block table.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call anything in oracle/.  The
product path never does, and this package imports nothing from it.

What it computes (llminference.xinbetween.com S06 "PagedAttention", section
"Implementation", the paged_attention excerpt; aicassindra.com
"tm_paged_attention_deep", section "The block table: logical to physical
mapping"):

  for every sequence s with L = context_lens[s] tokens,
    gather the logical keys/values: token t lives in physical block
      table[s][t // B] at offset t % B,
    and for every query head h, with its KV head g = h // (Hq / Hkv):
      z_t  = scale * <q[s, h], K_t[g]>
      w_t  = exp(z_t - max_t z_t)
      out  = sum_t w_t V_t[g] / sum_t w_t

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * query head h reads KV head h // (Hq / Hkv) (contiguous groups);
  * L counts the token appended this step;
  * L = 0 yields an all-zero output;
  * the printed excerpt's score line, q @ k_blk.transpose(0, 2, 1), does not
    give per-head scores for a [n, Hkv, D] block; read as a per-head dot
    product;
  * plain max-subtracted softmax, no mask beyond L.

Inputs are exact host copies: bfloat16 arrives as uint16 bit patterns and is
widened exactly (bits << 16 -> float32 -> float64); float32 widens exactly.
The scale is taken as float64(float32(scale)), the value the kernel receives.
Split-K partitioning is not modelled: merging per-partition softmax states by
log-sum-exp is an exact identity, so any partitioning must agree with this
unsplit definition within rounding.

Pinned by tests/test_oracle_pins.py (closed forms, brute force, a library
attention routine on the contiguous layout, permutation invariance, shared vs
private copies).
"""
from __future__ import annotations

import numpy as np


def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 copy of float32 data or of bfloat16 bit patterns (uint16)."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype == np.float32:
        return x.astype(np.float64)
    if x.dtype == np.float64:
        return x
    raise TypeError(f"unsupported dtype {x.dtype}")


def gather_logical(pool: np.ndarray, table_row: np.ndarray, length: int,
                   block_size: int) -> np.ndarray:
    """Logical rows 0..length-1 of one sequence, read through its table.

    Position t sits in physical block table_row[t // B] at offset t % B
    (synapticradio.com "The KV Cache Is an Allocator Problem", the
    physical-address equation in "What the trace shows").
    Returns the pool's dtype, shape [length, Hkv, D].
    """
    t = np.arange(length)
    logical_block = t // block_size
    offset = t % block_size
    n_blocks = pool.shape[0]
    phys = np.asarray(table_row)[logical_block]
    if length and (phys.min() < 0 or phys.max() >= n_blocks):
        raise ValueError("block table names a block outside the pool")
    return pool[phys, offset]


def attend(q_s: np.ndarray, keys: np.ndarray, values: np.ndarray,
           scale: float) -> np.ndarray:
    """Softmax attention of one sequence's queries over its logical K/V.

    q_s [Hq, D], keys/values [L, Hkv, D], all float64.  Returns [Hq, D].
    """
    hq, d = q_s.shape
    length, hkv, _ = keys.shape
    out = np.zeros((hq, d), dtype=np.float64)
    if length == 0:
        return out
    group = hq // hkv
    for h in range(hq):
        g = h // group
        z = scale * (keys[:, g, :] @ q_s[h])
        w = np.exp(z - z.max())
        out[h] = (w @ values[:, g, :]) / w.sum()
    return out


def decode_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                     block_tables: np.ndarray, context_lens: np.ndarray,
                     scale: float, seqs=None) -> np.ndarray:
    """Paged decode attention in float64.

    q [S, Hq, D]; k_pool/v_pool [NB, B, Hkv, D]; block_tables [S, max_blocks];
    context_lens [S].  `seqs` optionally restricts the work to some sequences
    (rows of the result for other sequences stay zero).  Returns [S, Hq, D].
    """
    num_seqs, hq, d = q.shape
    nb, block_size, hkv, d2 = k_pool.shape
    if d2 != d or v_pool.shape != k_pool.shape or hq % hkv:
        raise ValueError("shape mismatch")
    scale64 = float(np.float32(scale))
    out = np.zeros((num_seqs, hq, d), dtype=np.float64)
    for s in (range(num_seqs) if seqs is None else seqs):
        length = int(context_lens[s])
        if length < 0 or length > block_tables.shape[1] * block_size:
            raise ValueError("context length outside the table")
        keys = widen(gather_logical(k_pool, block_tables[s], length, block_size))
        values = widen(gather_logical(v_pool, block_tables[s], length, block_size))
        out[s] = attend(widen(q[s]), keys, values, scale64)
    return out
