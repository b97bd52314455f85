"""CPU oracle for the cache-writing operations, swapping and slot addressing.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call anything in oracle/.

Both operations are pure byte moves, so the oracle works on whatever array the
caller holds (float32 or bfloat16 bit patterns) and never converts values.
"""
from __future__ import annotations

import numpy as np


def slot_address(table_row, t: int, block_size: int) -> int:
    """Flat slot of logical position t: table[t // B] * B + t % B.

    synapticradio.com "The KV Cache Is an Allocator Problem", the
    physical-address equation under "What the trace shows"; the same mapping is
    stated as logical_block = t // B, offset = t % B on aicassindra.com
    "tm_paged_attention_deep", "The block table: logical to physical mapping".
    """
    return int(table_row[t // block_size]) * block_size + t % block_size


def reshape_and_cache(k_pool: np.ndarray, v_pool: np.ndarray, key: np.ndarray,
                      value: np.ndarray, slot_mapping: np.ndarray) -> None:
    """Write token i's key/value rows into flat slot slot_mapping[i]; skip < 0.

    The cache write of mercemay.com "Paged KV Cache Allocation and the Block
    Table", section "Blocks, tables, and the indirection": the slot
    physical * block_size + offset of the pool receives k (and v).
    Pools are [NB, B, Hkv, D]; key/value are [N, Hkv, D].  Modified in place.
    """
    nb, b, hkv, d = k_pool.shape
    k_flat = k_pool.reshape(nb * b, hkv, d)
    v_flat = v_pool.reshape(nb * b, hkv, d)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    if np.any(slots[keep] >= nb * b):
        raise ValueError("slot outside the pool")
    if len(np.unique(slots[keep])) != int(keep.sum()):
        raise ValueError("duplicate slots in one call")
    k_flat[slots[keep]] = key[keep]
    v_flat[slots[keep]] = value[keep]


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs: np.ndarray) -> None:
    """Copy-on-write duplication: pool[dst] = pool[src] for every (src, dst).

    Whole blocks, keys and values (aicassindra.com "tm_paged_attention_deep",
    "Copy-on-write for shared prefixes": the single block at the point of
    divergence is copied for the writer).  Modified in place.
    """
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    dsts = set(pairs[:, 1].tolist())
    if len(dsts) != len(pairs) or dsts & set(pairs[:, 0].tolist()):
        raise ValueError("destinations must be distinct and never a source")
    for src, dst in pairs:
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]


def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                pairs: np.ndarray) -> None:
    """Swap copy between a device pool and a host pool: dst[d] = src[s] for
    every (s, d), keys and values, whole blocks, bytes unchanged.

    The preemption option of copying a sequence's cache out to host memory and
    back instead of recomputing it (mercemay.com "Paged KV Cache Allocation
    and the Block Table", "Three ways contiguous reservation loses memory";
    llminference.xinbetween.com S06, third exercise).  The two pools share the
    per-block shape [B, Hkv, D]; their block counts may differ.  Modified in
    place.
    """
    if src_k.shape[1:] != dst_k.shape[1:] or src_k.dtype != dst_k.dtype:
        raise ValueError("pools must share block shape and dtype")
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if len(set(pairs[:, 1].tolist())) != len(pairs):
        raise ValueError("destinations must be distinct")
    if len(pairs) and (pairs[:, 0].min() < 0 or pairs[:, 0].max() >= len(src_k)
                       or pairs[:, 1].min() < 0 or pairs[:, 1].max() >= len(dst_k)):
        raise ValueError("block id outside its pool")
    for s, d in pairs:
        dst_k[d] = src_k[s]
        dst_v[d] = src_v[s]
