"""paged_kv_cache_115_amd: paged-KV-cache decode attention for MI355X.

Thin Python binding over libpagedkv.so (C ABI declared in include/pagedkv.h).
Every computation runs in the library: this module only marshals torch
tensors (device memory) and numpy arrays (host memory) into pointers and
sizes.  Importing it loads the library and fails loudly when it has not been
built (python -m paged_kv_cache_115_amd.build).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from ._lib import (LIB_PATH, PA_BF16, PA_DECODE_FIRST_BLOCKS, PA_DECODE_SHARED_KV, PA_F32, PA_JOB_SHARED, PA_JOB_WIDE, PA_SWAP_ENGINE_MEMCPY,
                   PA_SWAP_ENGINE_KERNEL, PA_SWAP_IN, PA_SWAP_OUT, PaDecodePlanInfo, PaError, PaKvPool, lib)

__all__ = [
    "set_debug", "validate_slots", "validate_copy_pairs", "validate_decode",
    "LIB_PATH", "PA_F32", "PA_BF16", "PA_DECODE_SHARED_KV", "PA_DECODE_FIRST_BLOCKS", "PA_JOB_SHARED", "PA_JOB_WIDE", "PaError", "BlockManager", "KvPool",
    "reshape_and_cache", "copy_blocks", "decode_plan", "decode_workspace_bytes",
    "decode", "decode_noalloc", "DecodePlan", "default_workgroups", "HostKvPool", "swap_blocks", "PA_SWAP_OUT", "PA_SWAP_IN",
    "PA_SWAP_ENGINE_KERNEL", "PA_SWAP_ENGINE_MEMCPY",
]


# Debug mode: before each GPU call, validate the contents of its device
# inputs on host copies (pa_validate_*): slots, copy pairs, table entries,
# lengths against the plan.  It copies those inputs to the host and therefore
# synchronizes; off unless PAGEDKV_DEBUG=1 or set_debug(True).
_debug = os.environ.get("PAGEDKV_DEBUG", "0") not in ("", "0")


def set_debug(on: bool) -> None:
    """Turn host-side validation of device inputs before every call on or off."""
    global _debug
    _debug = bool(on)


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib.pa_last_error().decode(errors="replace")
        raise PaError(status, f"{what}: {msg}")


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


class KvPool:
    """One layer's K and V pools: caller-owned device tensors [NB, B, Hkv, D]."""

    def __init__(self, k, v):
        if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4:
            raise ValueError("k and v pools must share a 4-D shape and dtype")
        if not (k.is_cuda and v.is_cuda and k.is_contiguous() and v.is_contiguous()):
            raise ValueError("pools must be contiguous device tensors")
        self.k, self.v = k, v
        nb, b, hkv, d = k.shape
        self.c = PaKvPool(_ptr(k), _ptr(v), nb, b, hkv, d, _dtype_code(k))

    @property
    def block_size(self) -> int:
        return self.c.block_size


class HostKvPool:
    """Swap space for one layer: caller-owned PINNED host tensors [NH, B, Hkv, D]
    with the device pool's block shape and dtype (torch.empty(..., pin_memory=True))."""

    def __init__(self, k, v):
        if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4:
            raise ValueError("k and v host pools must share a 4-D shape and dtype")
        if k.is_cuda or v.is_cuda or not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("host pools must be contiguous host tensors")
        if not (k.is_pinned() and v.is_pinned()):
            raise ValueError("host pools must be pinned (pin_memory=True)")
        self.k, self.v = k, v
        nb, b, hkv, d = k.shape
        self.c = PaKvPool(_ptr(k), _ptr(v), nb, b, hkv, d, _dtype_code(k))


def swap_blocks(pool: KvPool, host: HostKvPool, pairs, direction: int, engine: int = PA_SWAP_ENGINE_KERNEL,
                stream=None) -> None:
    """pa_swap_blocks: copy blocks between the device pool and the host pool.
    `pairs` is a host int32 array [n, 2] of (src, dst); PA_SWAP_OUT copies
    device -> host, PA_SWAP_IN host -> device.  Ordered on `stream`."""
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    n = pairs.shape[0]
    _check(lib.pa_swap_blocks(ctypes.byref(pool.c), ctypes.byref(host.c),
                              pairs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if n else None, n,
                              direction, engine, _stream(stream)), "pa_swap_blocks")


def _dev(t, name, dtype=None):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _host_i32(a):
    return np.ascontiguousarray(a.cpu().numpy() if hasattr(a, "cpu") else a, dtype=np.int32)


def validate_slots(pool: KvPool, slot_mapping) -> None:
    """pa_validate_slots on a host copy of a slot mapping (raises PaError)."""
    slots = np.ascontiguousarray(slot_mapping.cpu().numpy() if hasattr(slot_mapping, "cpu") else slot_mapping,
                                 dtype=np.int64)
    _check(lib.pa_validate_slots(slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), slots.size,
                                 pool.c.num_blocks, pool.c.block_size), "pa_validate_slots")


def validate_copy_pairs(pool: KvPool, pairs) -> None:
    """pa_validate_copy_pairs on a host copy of (src, dst) pairs (raises PaError)."""
    pr = _host_i32(pairs).reshape(-1)
    _check(lib.pa_validate_copy_pairs(pr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), pr.size // 2,
                                      pool.c.num_blocks), "pa_validate_copy_pairs")


def validate_decode(pool: KvPool, block_tables, context_lens, plan: "DecodePlan", fused_append: bool = False) -> None:
    """pa_validate_decode on host copies of a decode call's tables and lengths
    and the plan's host bytes (raises PaError)."""
    tables = _host_i32(block_tables)
    lens = _host_i32(context_lens).reshape(-1)
    if tables.ndim != 2 or tables.shape[0] != lens.size:
        raise ValueError("block_tables must be [num_seqs, max_blocks] with one length per row")
    _check(lib.pa_validate_decode(ctypes.byref(pool.c), tables.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  tables.shape[1], lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), lens.size,
                                  ctypes.c_void_p(plan.blob.ctypes.data), ctypes.byref(plan.info),
                                  int(bool(fused_append))), "pa_validate_decode")


def reshape_and_cache(pool: KvPool, key, value, slot_mapping, stream=None) -> None:
    """pa_reshape_and_cache: write key[i]/value[i] at flat slot slot_mapping[i]."""
    import torch
    _dev(key, "key", pool.k.dtype)
    _dev(value, "value", pool.k.dtype)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    n = slot_mapping.numel()
    if key.shape[0] != n or value.shape[0] != n or tuple(key.shape[1:]) != tuple(pool.k.shape[2:]):
        raise ValueError("key/value must be [num_tokens, Hkv, D] matching slot_mapping")
    if _debug:
        validate_slots(pool, slot_mapping)
    _check(lib.pa_reshape_and_cache(ctypes.byref(pool.c), _ptr(key), _ptr(value), _ptr(slot_mapping),
                                    n, _stream(stream)), "pa_reshape_and_cache")


def copy_blocks(pool: KvPool, pairs, stream=None) -> None:
    """pa_copy_blocks: for each (src, dst) row of int32 device `pairs`, dst := src."""
    import torch
    _dev(pairs, "pairs", torch.int32)
    n = pairs.numel() // 2
    if _debug:
        validate_copy_pairs(pool, pairs)
    _check(lib.pa_copy_blocks(ctypes.byref(pool.c), _ptr(pairs) if n else None, n, _stream(stream)),
           "pa_copy_blocks")


class DecodePlan:
    """Host-built schedule for one batch (pa_decode_plan).  `blob` is the plan
    bytes to copy to the device; `info` describes them."""

    JOB_FIELDS = ("seq", "tile_begin", "tile_count", "head_block", "part", "num_parts", "record_base", "reserved")

    def __init__(self, blob: np.ndarray, info: PaDecodePlanInfo):
        self.blob = blob          # uint8 [info.bytes]
        self.info = info

    def __getattr__(self, name):
        if name in ("num_workgroups", "num_jobs", "num_merges", "num_records", "num_kv_heads", "jobs_per_workgroup",
                    "schedule", "num_groups", "group_size"):
            return getattr(self.info, name)
        raise AttributeError(name)

    def job_table(self) -> np.ndarray:
        """int32 [jobs_per_workgroup, num_workgroups, 8]: slot k of workgroup b
        at [k, b]; empty slots have tile_count (field 2) 0."""
        n = self.info.jobs_per_workgroup * self.info.num_workgroups
        return self.blob[self.info.jobs_at:self.info.jobs_at + 32 * n].view(np.int32).reshape(
            self.info.jobs_per_workgroup, self.info.num_workgroups, 8)

    def jobs(self) -> np.ndarray:
        """int32 [num_jobs, 8]: seq, tile_begin, tile_count, head_block, part, num_parts, record_base, context_len;
        workgroup after workgroup, each in its processing order."""
        t = self.job_table().transpose(1, 0, 2).reshape(-1, 8)
        return t[t[:, 2] > 0]

    def groups(self) -> np.ndarray:
        """int32 [num_groups, 16]: num_members, head_block, seq[4], record_base[4], num_parts[4], 0, 0."""
        n = self.info.num_groups
        return self.blob[self.info.groups_at:self.info.groups_at + 64 * n].view(np.int32).reshape(n, 16)

    def merges(self) -> np.ndarray:
        """int32 [num_merges, 4]: seq, kv_head, num_parts, record_base."""
        n = self.info.num_merges
        return self.blob[self.info.merges_at:self.info.merges_at + 16 * n].view(np.int32).reshape(n, 4)

    def set_first_blocks(self, tables, block_size: int) -> "DecodePlan":
        """pa_decode_plan_first_blocks: write each job's first-tile table
        entries from the host tables (int32 [num_seqs, max_blocks]) that
        pa_decode will read; returns self."""
        tables = np.ascontiguousarray(tables, dtype=np.int32)
        if tables.ndim != 2:
            raise ValueError("tables must be [num_seqs, max_blocks]")
        _check(lib.pa_decode_plan_first_blocks(self.blob.ctypes.data_as(ctypes.c_void_p), ctypes.byref(self.info),
                                               tables.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                               tables.shape[1], tables.shape[0], block_size),
               "pa_decode_plan_first_blocks")
        return self

    def first_blocks(self) -> np.ndarray:
        """int32 [jobs_per_workgroup, num_workgroups, 4]: first-tile table entries."""
        n = self.info.jobs_per_workgroup * self.info.num_workgroups
        return self.blob[self.info.first_at:self.info.first_at + 16 * n].view(np.int32).reshape(
            self.info.jobs_per_workgroup, self.info.num_workgroups, 4)

    def check_lens(self, context_lens) -> None:
        """pa_decode_plan_check_lens: raise PaError unless the plan was made for
        exactly these (host) context lengths."""
        lens = _host_i32(context_lens).reshape(-1)
        _check(lib.pa_decode_plan_check_lens(ctypes.byref(self.info), lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                             lens.size), "pa_decode_plan_check_lens")

    def advance(self, context_lens, max_job_tiles: int = 0) -> bool:
        """pa_decode_plan_advance: carry this plan (in place) to the next
        step's lengths.  False, with the plan unchanged, when it cannot follow
        them (build a new plan then); the first-tile entries are dropped."""
        lens = _host_i32(context_lens).reshape(-1)
        if not self.blob.flags.writeable:
            raise ValueError("plan bytes are read-only")
        st = lib.pa_decode_plan_advance(ctypes.c_void_p(self.blob.ctypes.data), ctypes.byref(self.info),
                                        lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), lens.size,
                                        int(max_job_tiles))
        if st == PA_REPLAN:
            return False
        _check(st, "pa_decode_plan_advance")
        return True

    def to_device(self, device="cuda"):
        import torch
        return torch.from_numpy(self.blob.copy()).to(device)


# Host buffer the plan is built in (grown on demand); each DecodePlan copies
# its bytes out.
_plan_buf = np.zeros(1 << 13, dtype=np.uint64).view(np.uint8)


def default_workgroups() -> int:
    """Persistent decode workgroups filling the current device."""
    n = lib.pa_decode_default_workgroups()
    if n <= 0:
        raise PaError(-5, "pa_decode_default_workgroups: " + lib.pa_last_error().decode())
    return n


SCHEDULE_AUTO, SCHEDULE_CHUNKS, SCHEDULE_LPT = -1, 0, 1
PA_REPLAN = 1  # pa_decode_plan_advance: build a new plan


def _piece_cap(max_piece_tiles: int, block_size: int | None) -> int:
    """Longest job in tiles: pools of fewer than 8 slots per block take jobs
    of at most 8 * B tiles (the kernels' table window)."""
    if block_size is not None and block_size < 8:
        return min(max_piece_tiles, 8 * block_size) if max_piece_tiles > 0 else 8 * block_size
    return max_piece_tiles


def decode_plan(context_lens, num_kv_heads: int, num_workgroups: int | None = None,
                max_piece_tiles: int = 0, shared_kv: bool = False, schedule: int = SCHEDULE_AUTO,
                block_size: int | None = None) -> DecodePlan:
    """pa_decode_plan_schedule (pa_decode_plan for the automatic choice).
    num_workgroups defaults to default_workgroups().  shared_kv sets
    PA_DECODE_SHARED_KV: pass True when sequences of the batch share blocks
    (forked prefixes), so K/V loads keep them cached.  block_size: the pool's
    B; below 8 it caps pieces at 8 * B tiles, as pa_decode requires."""
    max_piece_tiles = _piece_cap(max_piece_tiles, block_size)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    if num_workgroups is None:
        num_workgroups = default_workgroups()
    info = PaDecodePlanInfo()
    p32 = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    global _plan_buf
    for _ in range(2):
        buf = _plan_buf
        st = lib.pa_decode_plan_schedule(p32, lens.size, num_kv_heads, num_workgroups, max_piece_tiles, schedule,
                                         ctypes.c_void_p(buf.ctypes.data), buf.size, ctypes.byref(info))
        if st == 0 or info.bytes <= buf.size:
            break
        _plan_buf = np.zeros(2 * info.bytes, dtype=np.uint64).view(np.uint8)   # 8-byte aligned
    _check(st, "pa_decode_plan_schedule")
    info.flags = PA_DECODE_SHARED_KV if shared_kv else 0
    return DecodePlan(buf[: info.bytes].copy(), info)


def decode_plan_prefix(context_lens, num_kv_heads: int, num_q_heads: int, prefix_group, prefix_tokens,
                       num_workgroups: int | None = None, max_piece_tiles: int = 0,
                       block_size: int | None = None) -> DecodePlan:
    """pa_decode_plan_prefix: shared prefixes read once per group (cascade
    decode).  prefix_group/prefix_tokens as from BlockManager.prefix_groups.
    The plan carries PA_DECODE_SHARED_KV only when some shared block is still
    read by more than one job (see pa_decode_plan_prefix).  block_size as for
    decode_plan."""
    max_piece_tiles = _piece_cap(max_piece_tiles, block_size)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    grp = np.ascontiguousarray(prefix_group, dtype=np.int32)
    tok = np.ascontiguousarray(prefix_tokens, dtype=np.int32)
    if grp.shape != lens.shape or tok.shape != lens.shape:
        raise ValueError("prefix_group and prefix_tokens must have one entry per sequence")
    if num_workgroups is None:
        num_workgroups = default_workgroups()
    info = PaDecodePlanInfo()
    p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    global _plan_buf
    for _ in range(2):
        buf = _plan_buf
        st = lib.pa_decode_plan_prefix(p32(lens), lens.size, num_kv_heads, num_q_heads, num_workgroups,
                                       max_piece_tiles, p32(grp), p32(tok), ctypes.c_void_p(buf.ctypes.data),
                                       buf.size, ctypes.byref(info))
        if st == 0 or info.bytes <= buf.size:
            break
        _plan_buf = np.zeros(2 * info.bytes, dtype=np.uint64).view(np.uint8)   # 8-byte aligned
    _check(st, "pa_decode_plan_prefix")
    return DecodePlan(buf[: info.bytes].copy(), info)


FUSED_LOADS = {0: "none (no fused append)", 1: "separate path for the appended token's tile",
               2: "per-lane addresses for every tile", 4: "buffer loads in a window holding pool and new rows"}


def decode_fused_loads(pool: KvPool, new_key, new_value, plan: DecodePlan, num_q_heads: int) -> int:
    """pa_decode_fused_loads: how pa_decode loads tiles for these arguments
    (see FUSED_LOADS); new_key/new_value are tensors or None."""
    nk = ctypes.c_void_p(new_key.data_ptr()) if new_key is not None else None
    nv = ctypes.c_void_p(new_value.data_ptr()) if new_value is not None else None
    m = lib.pa_decode_fused_loads(ctypes.byref(pool.c), nk, nv, plan.info.num_seqs, num_q_heads, ctypes.byref(plan.info))
    if m < 0:
        _check(-1, "pa_decode_fused_loads")
    return int(m)


def decode_workspace_bytes(plan: DecodePlan, num_q_heads: int, head_dim: int) -> int:
    return int(lib.pa_decode_workspace_bytes(ctypes.byref(plan.info), num_q_heads, head_dim))


_DECODE_STAGES = {"all": "pa_decode", "attention": "pa_decode_attention", "merge": "pa_decode_merge_pieces"}


def _decode_checked(pool: KvPool, q, block_tables, context_lens, plan: DecodePlan, plan_dev, out, new_key,
                    new_value) -> tuple:
    """Checks shared by the decode entry points; returns (S, Hq, out)."""
    import torch
    # The C ABI receives no head_dim for q, out or the new rows and no row
    # counts for the tables and lengths: shapes are checked here against the
    # pool, before anything else.
    if q.dim() != 3:
        raise ValueError("q must be [S, Hq, D]")
    s, hq, d = q.shape
    if d != pool.k.shape[3]:
        raise ValueError(f"q has head_dim {d}, the pool {pool.k.shape[3]}")
    if block_tables.dim() != 2 or block_tables.shape[0] != s:
        raise ValueError(f"block_tables must be [S={s}, max_blocks]")
    if context_lens.numel() != s:
        raise ValueError(f"context_lens must hold S={s} lengths")
    if out is not None and tuple(out.shape) != (s, hq, d):
        raise ValueError("out must be [S, Hq, D]")
    for t, n in ((new_key, "new_key"), (new_value, "new_value")):
        if t is not None and tuple(t.shape) != (s, pool.k.shape[2], d):
            raise ValueError(f"{n} must be [S, Hkv, D]")
    _dev(q, "q", pool.k.dtype)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    _dev(plan_dev, "plan_dev", torch.uint8)
    if plan_dev.numel() < plan.info.bytes:
        raise ValueError("plan_dev is shorter than the plan")
    if out is None:
        out = torch.empty((s, hq, d), dtype=torch.float32, device=q.device)
    _dev(out, "out")
    if out.dtype not in (torch.float32, pool.k.dtype):
        raise TypeError("out must be float32 or the pool dtype")
    if (new_key is None) != (new_value is None):
        raise ValueError("new_key and new_value go together")
    if new_key is not None:
        _dev(new_key, "new_key", pool.k.dtype)
        _dev(new_value, "new_value", pool.k.dtype)
    if _debug:
        validate_decode(pool, block_tables, context_lens, plan, fused_append=new_key is not None)
    return s, hq, out


def decode(pool: KvPool, q, block_tables, context_lens, scale: float, plan: DecodePlan, plan_dev, workspace=None,
           out=None, stream=None, stage: str = "all", new_key=None, new_value=None):
    """pa_decode (stage "all"), or one of its two launches: pa_decode_attention
    ("attention") or pa_decode_merge_pieces ("merge").  `plan_dev` is the device copy
    of plan.blob (uint8 tensor).  new_key/new_value ([S, Hkv, D], pool dtype)
    fuse this step's append: token L - 1 of every sequence is read from them
    and stored into its slot."""
    s, hq, out = _decode_checked(pool, q, block_tables, context_lens, plan, plan_dev, out, new_key, new_value)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = _DECODE_STAGES[stage]
    _check(getattr(lib, fn)(ctypes.byref(pool.c), _ptr(q), _ptr(out), _dtype_code(out), _ptr(block_tables),
                         block_tables.shape[1], _ptr(context_lens), s, hq, ctypes.c_float(scale),
                         None if new_key is None else _ptr(new_key), None if new_value is None else _ptr(new_value),
                         _ptr(plan_dev),
                         ctypes.byref(plan.info), None if workspace is None else _ptr(workspace), ws_bytes,
                         _stream(stream)), fn)
    return out


def decode_noalloc(pool: KvPool, q, block_tables, context_lens, scale: float, plan: DecodePlan, plan_dev, out,
                   stream=None, new_key=None, new_value=None):
    """pa_decode_noalloc: pa_decode with the library's built-in scratch array
    (PA_NOALLOC_SCRATCH_BYTES per device) as its workspace; allocates
    nothing, so `out` must be given.  Calls on one device share the array:
    order them on one stream."""
    if out is None:
        raise ValueError("decode_noalloc allocates nothing: pass out")
    s, hq, out = _decode_checked(pool, q, block_tables, context_lens, plan, plan_dev, out, new_key, new_value)
    _check(lib.pa_decode_noalloc(ctypes.byref(pool.c), _ptr(q), _ptr(out), _dtype_code(out), _ptr(block_tables),
                                 block_tables.shape[1], _ptr(context_lens), s, hq, ctypes.c_float(scale),
                                 None if new_key is None else _ptr(new_key),
                                 None if new_value is None else _ptr(new_value), _ptr(plan_dev),
                                 ctypes.byref(plan.info), _stream(stream)), "pa_decode_noalloc")
    return out


def probe_read(src, num_workgroups: int, sink, nbytes: int | None = None, stream=None) -> None:
    """pa_probe_read: stream-read nbytes (default: all) of device tensor src
    once; sink is a device tensor of at least num_workgroups * 256 uint32."""
    _dev(src, "src")
    _dev(sink, "sink")
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > src.numel() * src.element_size() or sink.numel() * sink.element_size() < 4 * 256 * num_workgroups:
        raise ValueError("probe_read: nbytes past src or sink too small")
    _check(lib.pa_probe_read(_ptr(src), n, num_workgroups, _ptr(sink), _stream(stream)), "pa_probe_read")


class BlockManager:
    """Host block manager (pa_bm_*): free list, tables, counts, copy-on-write."""

    def __init__(self, num_blocks: int, block_size: int, initial_order=None):
        order = None
        if initial_order is not None:
            order = np.ascontiguousarray(initial_order, dtype=np.int32)
            if order.size != num_blocks:
                raise ValueError("initial_order must list every block once")
        self._order = order
        ptr = None if order is None else order.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        self._h = lib.pa_bm_create(num_blocks, block_size, ptr)
        if not self._h:
            raise PaError(-1, "pa_bm_create: " + lib.pa_last_error().decode())
        self.num_blocks = num_blocks
        self.block_size = block_size

    # Bound once, so that a manager collected at interpreter shutdown (after
    # module globals are cleared) can still release its handle.
    _destroy = staticmethod(lib.pa_bm_destroy)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._destroy(h)
            self._h = None

    def append(self, seq: int, n_new: int = 1):
        """Returns (slots int64[n_new], cow pairs int32[k, 2])."""
        slots = np.zeros(max(n_new, 1), dtype=np.int64)
        cow = np.zeros(2, dtype=np.int32)
        n_cow = ctypes.c_int32(0)
        _check(lib.pa_bm_append(self._h, seq, n_new, slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                cow.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(n_cow)),
               "pa_bm_append")
        return slots[:n_new], cow[: 2 * n_cow.value].reshape(-1, 2)

    def append_step(self, seqs):
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = seqs.size
        slots = np.zeros(max(n, 1), dtype=np.int64)
        cow = np.zeros(max(2 * n, 2), dtype=np.int32)
        n_cow = ctypes.c_int32(0)
        _check(lib.pa_bm_append_step(self._h, seqs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n,
                                     slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     cow.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(n_cow)),
               "pa_bm_append_step")
        return slots[:n], cow[: 2 * n_cow.value].reshape(-1, 2)

    def fork(self, parent: int, child: int) -> None:
        _check(lib.pa_bm_fork(self._h, parent, child), "pa_bm_fork")

    def free(self, seq: int) -> None:
        _check(lib.pa_bm_free(self._h, seq), "pa_bm_free")

    def table(self, seq: int) -> np.ndarray:
        n = lib.pa_bm_table(self._h, seq, None, 0)
        if n < 0:
            raise KeyError(seq)
        out = np.zeros(max(n, 1), dtype=np.int32)
        lib.pa_bm_table(self._h, seq, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n)
        return out[:n]

    def prefix_groups(self, seqs):
        """pa_bm_prefix_groups -> (group int32[n], prefix_tokens int32[n])."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        group = np.zeros(seqs.size, dtype=np.int32)
        tokens = np.zeros(seqs.size, dtype=np.int32)
        _check(lib.pa_bm_prefix_groups(self._h, seqs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), seqs.size,
                                       group.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                       tokens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))), "pa_bm_prefix_groups")
        return group, tokens

    def export(self, seqs, max_blocks: int):
        """Dense (tables int32[n, max_blocks], lens int32[n]) for upload."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        tables = np.zeros((seqs.size, max(max_blocks, 1)), dtype=np.int32)
        lens = np.zeros(seqs.size, dtype=np.int32)
        _check(lib.pa_bm_export(self._h, seqs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), seqs.size,
                                max_blocks, tables.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))), "pa_bm_export")
        return tables[:, :max_blocks] if max_blocks else tables[:, :0], lens

    def set_host_blocks(self, n: int) -> None:
        _check(lib.pa_bm_set_host_blocks(self._h, n), "pa_bm_set_host_blocks")

    def _swap(self, fn, seqs, what):
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        cap = 0
        for s in seqs.tolist():
            n = lib.pa_bm_table(self._h, s, None, 0)
            cap += max(n, 0)
        pairs = np.zeros((max(cap, 1), 2), dtype=np.int32)
        n_pairs = ctypes.c_int32(0)
        _check(fn(self._h, seqs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), seqs.size,
                  pairs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), cap, ctypes.byref(n_pairs)), what)
        return pairs[:n_pairs.value]

    def swap_out(self, seqs) -> np.ndarray:
        """pa_bm_swap_out -> int32 [n, 2] (device block, host block) copies."""
        return self._swap(lib.pa_bm_swap_out, seqs, "pa_bm_swap_out")

    def swap_in(self, seqs) -> np.ndarray:
        """pa_bm_swap_in -> int32 [n, 2] (host block, device block) copies."""
        return self._swap(lib.pa_bm_swap_in, seqs, "pa_bm_swap_in")

    def enable_prefix_cache(self) -> None:
        _check(lib.pa_bm_enable_prefix_cache(self._h), "pa_bm_enable_prefix_cache")

    def append_prompt(self, seq: int, tokens):
        """pa_bm_append_prompt -> (slots int64[n] with -1 for reused tokens, cached token count)."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        n = tokens.size
        slots = np.zeros(max(n, 1), dtype=np.int64)
        cached = ctypes.c_int32(0)
        _check(lib.pa_bm_append_prompt(self._h, seq, tokens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n,
                                       slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ctypes.byref(cached)),
               "pa_bm_append_prompt")
        return slots[:n], cached.value

    def is_cached(self, block: int) -> bool:
        return lib.pa_bm_cached(self._h, block) == 1

    def is_swapped(self, seq: int) -> bool:
        r = lib.pa_bm_swapped(self._h, seq)
        if r < 0:
            raise KeyError(seq)
        return bool(r)

    def host_refcount(self, block: int) -> int:
        return lib.pa_bm_host_refcount(self._h, block)

    def prepare_decode_step(self, seqs, max_blocks: int, num_kv_heads: int, buffer, num_workgroups: int | None = None,
                            schedule: int = -1, first_blocks: bool = True):
        """pa_bm_prepare_decode_step: append one token to each sequence and
        write slots, copy pairs, lengths, table rows and the plan for the new
        lengths into `buffer` (a 256-byte aligned host uint8 array or pinned
        tensor).  Returns (layout, DecodePlan whose blob views the buffer's
        plan bytes)."""
        from ._lib import PaDecodeStepLayout
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        arr = buffer.numpy() if hasattr(buffer, "numpy") else buffer
        if num_workgroups is None:
            num_workgroups = default_workgroups()
        lay = PaDecodeStepLayout()
        _check(lib.pa_bm_prepare_decode_step(self._h, seqs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), seqs.size,
                                             max_blocks, num_kv_heads, num_workgroups, schedule, int(first_blocks),
                                             ctypes.c_void_p(arr.ctypes.data), arr.nbytes, ctypes.byref(lay)),
               "pa_bm_prepare_decode_step")
        plan = DecodePlan(arr[lay.plan_at:lay.plan_at + lay.plan.bytes], PaDecodePlanInfo.from_buffer_copy(lay.plan))
        return lay, plan

    def set_plan_reuse(self, max_advances: int) -> None:
        """pa_bm_set_plan_reuse: let prepare_decode_step advance its last plan
        (pa_decode_plan_advance) up to max_advances steps in a row; 0 builds
        every step."""
        _check(lib.pa_bm_set_plan_reuse(self._h, int(max_advances)), "pa_bm_set_plan_reuse")

    def length(self, seq: int) -> int:
        n = lib.pa_bm_len(self._h, seq)
        if n < 0:
            raise KeyError(seq)
        return n

    def refcount(self, block: int) -> int:
        return lib.pa_bm_refcount(self._h, block)

    def stats(self) -> dict:
        from ._lib import PaBmStats
        st = PaBmStats()
        lib.pa_bm_get_stats(self._h, ctypes.byref(st))
        return {name: getattr(st, name) for name, _ in PaBmStats._fields_ if not name.endswith("_")}

    def check(self) -> None:
        _check(lib.pa_bm_check(self._h), "pa_bm_check")
