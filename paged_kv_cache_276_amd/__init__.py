"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

Thin binding over the C ABI of ``libpagedkv.so`` (``include/pagedkv.h``).  The
functions carry the C entry points' names and only marshal arguments: shape and
dtype checks, pointers, the current HIP stream, and a cached workspace buffer.
Every step of the computation runs in the library's HIP kernels; there is no
CPU or PyTorch fallback.

    paged_kv_write(k_new, v_new, slot_mapping, k_cache, v_cache)
    out = paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, scale)
    paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out)  # no allocation
    out = paged_attn_decode_prefix(q, k_cache, v_cache, block_tables, context_lens,
                                   seq_prefix_tokens, groups, max_prefix_tokens, scale)
    out = paged_attn_decode_multi(q, k_cache, v_cache, block_tables, context_lens,
                                  cu_q_lens, max_q_len, scale)       # several new tokens each
    paged_block_copy(k_cache, v_cache, pairs)      # copy-on-write of whole blocks
    BlockManager(num_blocks, block_size)           # host block manager (blocks.py)

Layouts: pools ``[num_blocks][num_kv_heads][block_size][head_dim]`` (fp32 or
bf16); ``q`` ``[num_seqs][num_q_heads][head_dim]`` of the pool dtype;
``block_tables`` int32 ``[num_seqs][max_blocks_per_seq]``; ``context_lens`` and
``slot_mapping`` int32; ``out`` fp32 ``[num_seqs][num_q_heads][head_dim]``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

from . import _lib
from .blocks import BlockManager  # noqa: F401
from ._lib import (  # noqa: F401
    KERNEL_NAMES,
    PKV_KERNEL_AUTO,
    PKV_KERNEL_FAST,
    PKV_KERNEL_GENERIC,
    CacheDesc,
    DecodeOpts,
    DecodePlan,
    PkvError,
)

__all__ = [
    "BlockManager",
    "paged_block_copy",
    "paged_kv_write",
    "paged_attn_decode",
    "paged_attn_decode_multi",
    "paged_attn_decode_noalloc",
    "paged_attn_decode_prefix",
    "paged_attn_multi_plan",
    "paged_attn_prefix_plan",
    "paged_attn_plan",
    "paged_attn_workspace_bytes",
    "cache_desc",
    "last_launch_info",
    "new_workspace",
    "version",
    "PkvError",
]

_DTYPES = {torch.float32: _lib.PKV_F32, torch.bfloat16: _lib.PKV_BF16}


def version() -> str:
    return _lib.lib().pkv_version().decode()


def last_launch_info() -> Dict[str, object]:
    """What this thread's last paged_attn_decode / paged_attn_decode_prefix call launched: kernel
    family, grid (fast: waves; generic: partition workgroups), the odd-XCD share used and the
    tokens per tile or partition."""
    info = _lib.LaunchInfo()
    _lib.check(_lib.lib().pkv_last_launch_info(ctypes.byref(info)), "pkv_last_launch_info")
    return {"kernel": _lib.KERNEL_NAMES.get(info.kernel, "none"), "grid": info.grid,
            "xcd_balance": info.xcd_balance, "partition_tokens": info.partition_tokens,
            "k_stream": bool(info.k_stream)}


def cache_desc(k_cache: torch.Tensor) -> CacheDesc:
    if k_cache.dim() != 4:
        raise ValueError("cache must be [num_blocks][num_kv_heads][block_size][head_dim]")
    if k_cache.dtype not in _DTYPES:
        raise ValueError(f"unsupported cache dtype {k_cache.dtype}")
    nb, hkv, b, d = k_cache.shape
    return CacheDesc(nb, b, hkv, d, _DTYPES[k_cache.dtype])


# Default share (in 64ths of an equal share) of the fast kernel's waves on odd-numbered XCDs;
# the same value as PKV_XCD_BALANCE_DEFAULT in include/pagedkv.h.
XCD_BALANCE_DEFAULT = 62


def _opts(partition_tokens: int, kernel: int, grid_waves: int = 0, xcd_balance: int = 0) -> DecodeOpts:
    return DecodeOpts(int(partition_tokens), int(kernel), int(grid_waves), int(xcd_balance))


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev(t: torch.Tensor, name: str, device: torch.device) -> None:
    _need(t.is_cuda, f"{name} must be a GPU tensor")
    _need(t.device == device, f"{name} is on {t.device}, expected {device}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def debug_enabled() -> bool:
    """PKV_DEBUG=1 in the environment turns on the binding's host-side content checks."""
    return os.environ.get("PKV_DEBUG", "") not in ("", "0")


def check_distinct_slots(slots) -> None:
    """Raise ValueError if two tokens name the same slot (negative slots are skipped, so they may
    repeat).  Two writes to one slot race in the kernel; the library does not check device
    contents, so this runs on a host copy when PKV_DEBUG is set."""
    import numpy as np

    s = np.asarray(slots).astype(np.int64).ravel()
    s = s[s >= 0]
    uniq, counts = np.unique(s, return_counts=True)
    if np.any(counts > 1):
        dup = uniq[counts > 1]
        tokens = np.nonzero(np.isin(np.asarray(slots).ravel(), dup[:1]))[0]
        raise ValueError(f"slot_mapping names {len(dup)} slot(s) more than once "
                         f"(slot {int(dup[0])} for tokens {tokens.tolist()})")


def paged_kv_write(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Store token t's K/V rows at slot slot_mapping[t] (negative = skip), bit-exact, in place.
    With PKV_DEBUG=1 the slots are first read back and checked to be distinct (a synchronising
    copy; ValueError on a repeat)."""
    dev = k_cache.device
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (slot_mapping, "slot_mapping"),
                 (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n, dev)
    desc = cache_desc(k_cache)
    _need(v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype, "k_cache/v_cache differ")
    _need(slot_mapping.dtype == torch.int32 and slot_mapping.dim() == 1, "slot_mapping must be int32 [T]")
    T = slot_mapping.shape[0]
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t.dtype == k_cache.dtype, f"{n} dtype must match the cache")
        _need(tuple(t.shape) == (T, desc.num_kv_heads, desc.head_dim), f"{n} must be [T][Hkv][D]")
    if debug_enabled():
        check_distinct_slots(slot_mapping.cpu().numpy())
    st = _lib.lib().paged_kv_write(
        ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
        ctypes.c_void_p(slot_mapping.data_ptr()), T, ctypes.c_void_p(k_cache.data_ptr()),
        ctypes.c_void_p(v_cache.data_ptr()), ctypes.byref(desc), _stream(dev, stream))
    _lib.check(st, "paged_kv_write")


def paged_block_copy(k_cache: torch.Tensor, v_cache: torch.Tensor, pairs: torch.Tensor, stream=None) -> None:
    """Copy whole blocks in both pools: block pairs[p][1] becomes block pairs[p][0], bit for bit."""
    dev = k_cache.device
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (pairs, "pairs")):
        _dev(t, n, dev)
    desc = cache_desc(k_cache)
    _need(v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype, "k_cache/v_cache differ")
    _need(pairs.dtype == torch.int32 and pairs.dim() == 2 and pairs.shape[1] == 2, "pairs must be int32 [n][2]")
    st = _lib.lib().paged_block_copy(ctypes.c_void_p(k_cache.data_ptr()), ctypes.c_void_p(v_cache.data_ptr()),
                                     ctypes.c_void_p(pairs.data_ptr()), pairs.shape[0], ctypes.byref(desc),
                                     _stream(dev, stream))
    _lib.check(st, "paged_block_copy")


def paged_attn_plan(num_seqs: int, num_q_heads: int, max_blocks_per_seq: int, cache,
                    partition_tokens: int = 0, kernel: int = PKV_KERNEL_AUTO,
                    grid_waves: int = 0, xcd_balance: int = 0) -> Dict[str, int]:
    """Host-only launch plan (kernel family, partition size, grid, workspace bytes)."""
    desc = cache if isinstance(cache, CacheDesc) else cache_desc(cache)
    plan = DecodePlan()
    st = _lib.lib().paged_attn_plan(num_seqs, num_q_heads, max_blocks_per_seq, ctypes.byref(desc),
                                    ctypes.byref(_opts(partition_tokens, kernel, grid_waves, xcd_balance)),
                                    ctypes.byref(plan))
    _lib.check(st, "paged_attn_plan")
    return {
        "kernel": KERNEL_NAMES.get(plan.kernel, str(plan.kernel)),
        "partition_tokens": plan.partition_tokens,
        "max_partitions": plan.max_partitions,
        "threads_per_block": plan.threads_per_block,
        "grid_blocks": plan.grid_blocks,
        "workspace_bytes": plan.workspace_bytes,
    }


def paged_attn_workspace_bytes(num_seqs: int, num_q_heads: int, max_blocks_per_seq: int, cache,
                               partition_tokens: int = 0, kernel: int = PKV_KERNEL_AUTO,
                               grid_waves: int = 0, xcd_balance: int = 0) -> int:
    desc = cache if isinstance(cache, CacheDesc) else cache_desc(cache)
    out = ctypes.c_uint64(0)
    st = _lib.lib().paged_attn_workspace_bytes(num_seqs, num_q_heads, max_blocks_per_seq,
                                               ctypes.byref(desc),
                                               ctypes.byref(_opts(partition_tokens, kernel, grid_waves, xcd_balance)),
                                               ctypes.byref(out))
    _lib.check(st, "paged_attn_workspace_bytes")
    return int(out.value)


# One cached workspace per (device, stream): calls on one stream are ordered, so
# they can share it.  It is zero-filled when allocated: its first
# PKV_WORKSPACE_COUNTER_BYTES are the arrival counters of paged_attn_decode_multi,
# which must start at zero (every call leaves them so).
_workspaces: Dict[Tuple[torch.device, int], torch.Tensor] = {}

WORKSPACE_COUNTER_BYTES = 65536 * 4  # PKV_WORKSPACE_COUNTER_BYTES of include/pagedkv.h


def new_workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    """A zero-filled workspace of at least `nbytes` bytes, ready when this returns (the fill is
    synchronised, so the workspace can be used on any stream)."""
    ws = torch.zeros(max(16, (nbytes + 15) // 16 * 16), dtype=torch.uint8, device=device)
    torch.cuda.synchronize(device)
    return ws


def _workspace(device: torch.device, stream_handle: int, nbytes: int) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    key = (device, stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = new_workspace(nbytes, device)
        _workspaces[key] = ws
    return ws


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, out):
    """Shape, dtype and device checks shared by the decode entry points; returns (desc, S, Hq, out)."""
    dev = k_cache.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (block_tables, "block_tables"), (context_lens, "context_lens")):
        _dev(t, n, dev)
    desc = cache_desc(k_cache)
    _need(v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype, "k_cache/v_cache differ")
    _need(q.dim() == 3 and q.shape[2] == desc.head_dim and q.dtype == k_cache.dtype,
          "q must be [S][Hq][D] of the cache dtype")
    S, Hq = q.shape[0], q.shape[1]
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == S,
          "block_tables must be int32 [S][max_blocks_per_seq]")
    _need(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (S,),
          "context_lens must be int32 [S]")
    if out is None:
        out = torch.empty((S, Hq, desc.head_dim), dtype=torch.float32, device=dev)
    _dev(out, "out", dev)
    _need(out.dtype == torch.float32 and tuple(out.shape) == (S, Hq, desc.head_dim), "out must be fp32 [S][Hq][D]")
    return desc, S, Hq, out


def paged_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      partition_tokens: int = 0, kernel: int = PKV_KERNEL_AUTO,
                      grid_waves: int = 0, xcd_balance: int = 0, stream=None) -> torch.Tensor:
    """out[i][h] = softmax(scale * q[i][h] . K_i^T) V_i over the paged K/V of sequence i (fp32)."""
    dev = k_cache.device
    desc, S, Hq, out = _decode_args(q, k_cache, v_cache, block_tables, context_lens, out)
    maxb = block_tables.shape[1]
    opts = _opts(partition_tokens, kernel, grid_waves, xcd_balance)
    s = _stream(dev, stream)
    plan = paged_attn_plan(S, Hq, maxb, desc, partition_tokens, kernel, grid_waves, xcd_balance)
    need = plan["workspace_bytes"]
    if workspace is None:
        workspace = _workspace(dev, int(s.value or 0), need)
    elif need:
        _dev(workspace, "workspace", dev)
        _need(workspace.numel() * workspace.element_size() >= need, f"workspace needs {need} bytes")
    ws_ptr = ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.lib().paged_attn_decode(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()),
        ctypes.c_void_p(v_cache.data_ptr()), ctypes.c_void_p(block_tables.data_ptr()), maxb,
        ctypes.c_void_p(context_lens.data_ptr()), S, Hq, ctypes.c_float(scale),
        ctypes.c_void_p(out.data_ptr()), ws_ptr, ws_bytes, ctypes.byref(desc), ctypes.byref(opts), s)
    _lib.check(st, "paged_attn_decode")
    return out


# Scratch bytes of the allocation-free entry point (PKV_NOALLOC_SCRATCH_BYTES in include/pagedkv.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def paged_attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                              out: torch.Tensor, partition_tokens: int = 0, kernel: int = PKV_KERNEL_AUTO,
                              grid_waves: int = 0, xcd_balance: int = 0, stream=None) -> torch.Tensor:
    """paged_attn_decode with the library's own device scratch instead of a workspace: nothing is
    allocated, `out` included (the caller passes it).  Calls that may overlap on one GPU race."""
    dev = k_cache.device
    desc, S, Hq, out = _decode_args(q, k_cache, v_cache, block_tables, context_lens, out)
    maxb = block_tables.shape[1]
    opts = _opts(partition_tokens, kernel, grid_waves, xcd_balance)
    st = _lib.lib().paged_attn_decode_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()),
        ctypes.c_void_p(v_cache.data_ptr()), ctypes.c_void_p(block_tables.data_ptr()), maxb,
        ctypes.c_void_p(context_lens.data_ptr()), S, Hq, ctypes.c_float(scale),
        ctypes.c_void_p(out.data_ptr()), ctypes.byref(desc), ctypes.byref(opts), _stream(dev, stream))
    _lib.check(st, "paged_attn_decode_noalloc")
    return out


def paged_attn_prefix_plan(num_seqs: int, num_q_heads: int, max_blocks_per_seq: int, num_groups: int,
                           max_prefix_tokens: int, cache, chunk_tokens: int = 0, grid_waves: int = 0,
                           xcd_balance: int = 0) -> Dict[str, int]:
    """Host-only plan of the shared-prefix decode (prefix chunk, chunks, workspace bytes)."""
    desc = cache if isinstance(cache, CacheDesc) else cache_desc(cache)
    plan = DecodePlan()
    st = _lib.lib().paged_attn_prefix_plan(num_seqs, num_q_heads, max_blocks_per_seq, num_groups,
                                           max_prefix_tokens, ctypes.byref(desc),
                                           ctypes.byref(_opts(chunk_tokens, PKV_KERNEL_AUTO, grid_waves, xcd_balance)),
                                           ctypes.byref(plan))
    _lib.check(st, "paged_attn_prefix_plan")
    return {"kernel": KERNEL_NAMES.get(plan.kernel, str(plan.kernel)), "chunk_tokens": plan.partition_tokens,
            "max_chunks": plan.max_partitions, "workspace_bytes": plan.workspace_bytes}


def paged_attn_decode_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             block_tables: torch.Tensor, context_lens: torch.Tensor,
                             seq_prefix_tokens: torch.Tensor, groups: torch.Tensor, max_prefix_tokens: int,
                             scale: float, out: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None, chunk_tokens: int = 0,
                             grid_waves: int = 0, xcd_balance: int = 0, stream=None) -> torch.Tensor:
    """paged_attn_decode for groups of sequences sharing prefix blocks; each shared block is read once per group."""
    dev = k_cache.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_tables, "block_tables"),
                 (context_lens, "context_lens"), (seq_prefix_tokens, "seq_prefix_tokens"), (groups, "groups")):
        _dev(t, n, dev)
    desc = cache_desc(k_cache)
    _need(v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype, "k_cache/v_cache differ")
    _need(q.dim() == 3 and q.shape[2] == desc.head_dim and q.dtype == k_cache.dtype,
          "q must be [S][Hq][D] of the cache dtype")
    S, Hq = q.shape[0], q.shape[1]
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == S,
          "block_tables must be int32 [S][max_blocks_per_seq]")
    for t, n in ((context_lens, "context_lens"), (seq_prefix_tokens, "seq_prefix_tokens")):
        _need(t.dtype == torch.int32 and tuple(t.shape) == (S,), f"{n} must be int32 [S]")
    _need(groups.dtype == torch.int32 and groups.dim() == 2 and groups.shape[1] == 2, "groups must be int32 [G][2]")
    if out is None:
        out = torch.empty((S, Hq, desc.head_dim), dtype=torch.float32, device=dev)
    _dev(out, "out", dev)
    _need(out.dtype == torch.float32 and tuple(out.shape) == (S, Hq, desc.head_dim), "out must be fp32 [S][Hq][D]")
    maxb = block_tables.shape[1]
    G = groups.shape[0]
    plan = paged_attn_prefix_plan(S, Hq, maxb, G, max_prefix_tokens, desc, chunk_tokens, grid_waves, xcd_balance)
    s = _stream(dev, stream)
    need = plan["workspace_bytes"]
    if workspace is None:
        workspace = _workspace(dev, int(s.value or 0), need)
    else:
        _dev(workspace, "workspace", dev)
        _need(workspace.numel() * workspace.element_size() >= need, f"workspace needs {need} bytes")
    st = _lib.lib().paged_attn_decode_prefix(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()), ctypes.c_void_p(v_cache.data_ptr()),
        ctypes.c_void_p(block_tables.data_ptr()), maxb, ctypes.c_void_p(context_lens.data_ptr()), S, Hq,
        ctypes.c_void_p(seq_prefix_tokens.data_ptr()), ctypes.c_void_p(groups.data_ptr()), G,
        int(max_prefix_tokens), ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), ctypes.byref(desc),
        ctypes.byref(_opts(chunk_tokens, PKV_KERNEL_AUTO, grid_waves, xcd_balance)), s)
    _lib.check(st, "paged_attn_decode_prefix")
    return out


def paged_attn_multi_plan(num_seqs: int, total_q: int, max_q_len: int, num_q_heads: int, max_blocks_per_seq: int,
                          cache, chunk_tokens: int = 0, grid_waves: int = 0) -> Dict[str, int]:
    """Host-only plan of the multi-token attention (context chunk, chunks, workgroups, workspace bytes).

    With one wave per row block (max_q_len * G <= 16) and chunk_tokens 0 the tiles are split in equal runs
    over the resident waves (or grid_waves waves): chunk_tokens is then 16 and workgroups the wave count
    asked for (0 = the device's resident waves)."""
    desc = cache if isinstance(cache, CacheDesc) else cache_desc(cache)
    plan = DecodePlan()
    st = _lib.lib().paged_attn_multi_plan(num_seqs, total_q, max_q_len, num_q_heads, max_blocks_per_seq,
                                          ctypes.byref(desc),
                                          ctypes.byref(_opts(chunk_tokens, PKV_KERNEL_AUTO, grid_waves)),
                                          ctypes.byref(plan))
    _lib.check(st, "paged_attn_multi_plan")
    return {"chunk_tokens": plan.partition_tokens, "max_chunks": plan.max_partitions,
            "workgroups": plan.grid_blocks, "workspace_bytes": plan.workspace_bytes}


def paged_attn_decode_multi(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor, cu_q_lens: torch.Tensor,
                            max_q_len: int, scale: float, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, chunk_tokens: int = 0,
                            grid_waves: int = 0, stream=None) -> torch.Tensor:
    """Causal attention of several new tokens per sequence over the paged cache (fp32 out [total_q][Hq][D])."""
    dev = k_cache.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_tables, "block_tables"),
                 (context_lens, "context_lens"), (cu_q_lens, "cu_q_lens")):
        _dev(t, n, dev)
    desc = cache_desc(k_cache)
    _need(v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype, "k_cache/v_cache differ")
    _need(q.dim() == 3 and q.shape[2] == desc.head_dim and q.dtype == k_cache.dtype,
          "q must be [total_q][Hq][D] of the cache dtype")
    TQ, Hq = q.shape[0], q.shape[1]
    S = context_lens.shape[0]
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == S,
          "block_tables must be int32 [S][max_blocks_per_seq]")
    _need(context_lens.dtype == torch.int32 and context_lens.dim() == 1, "context_lens must be int32 [S]")
    _need(cu_q_lens.dtype == torch.int32 and tuple(cu_q_lens.shape) == (S + 1,), "cu_q_lens must be int32 [S+1]")
    if out is None:
        out = torch.empty((TQ, Hq, desc.head_dim), dtype=torch.float32, device=dev)
    _dev(out, "out", dev)
    _need(out.dtype == torch.float32 and tuple(out.shape) == (TQ, Hq, desc.head_dim), "out must be fp32 [total_q][Hq][D]")
    maxb = block_tables.shape[1]
    plan = paged_attn_multi_plan(S, TQ, max_q_len, Hq, maxb, desc, chunk_tokens, grid_waves)
    s = _stream(dev, stream)
    need = plan["workspace_bytes"]
    if workspace is None:
        workspace = _workspace(dev, int(s.value or 0), need)
    else:
        _dev(workspace, "workspace", dev)
        _need(workspace.numel() * workspace.element_size() >= need, f"workspace needs {need} bytes")
    st = _lib.lib().paged_attn_decode_multi(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()), ctypes.c_void_p(v_cache.data_ptr()),
        ctypes.c_void_p(block_tables.data_ptr()), maxb, ctypes.c_void_p(context_lens.data_ptr()),
        ctypes.c_void_p(cu_q_lens.data_ptr()), S, TQ, int(max_q_len), Hq, ctypes.c_float(scale),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), ctypes.byref(desc),
        ctypes.byref(_opts(chunk_tokens, PKV_KERNEL_AUTO, grid_waves)), s)
    _lib.check(st, "paged_attn_decode_multi")
    return out
