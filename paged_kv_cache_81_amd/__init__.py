"""Paged KV cache decode path for AMD Instinct MI355X (gfx950).

Thin PyTorch-facing wrappers around the C ABI of ``libpagedkv.so``
(include/paged_kv.h).  They only check shapes, dtypes and devices and pass
``data_ptr()``s and the current HIP stream; every step of the computation runs
in the library's HIP kernels.  PyTorch provides device memory and streams.

Cache layout (one attention layer): ``kv_cache[2, num_blocks, block_size,
num_kv_heads, head_size]``, index 0 keys and index 1 values.
"""
from __future__ import annotations

import ctypes

from typing import Optional, Tuple

import torch

from ._lib import PKV_ATTN_CACHED_KV, PKV_BF16, PKV_F32, PagedKVError, check, lib

__all__ = ["slot_mapping", "write", "gather", "copy_blocks", "partition_size", "workspace_bytes",
           "attention_decode_append", "attention_append_partitions",
           "attention_decode", "attention_partitions", "attention_merge", "attention_prefill",
           "PagedKVError"]

_DTYPES = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported element type {t.dtype} (float32 or bfloat16)") from None


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _cache_dims(kv_cache: torch.Tensor):
    _need(kv_cache, "kv_cache", ndim=5)
    two, nb, b, hkv, d = kv_cache.shape
    if two != 2:
        raise ValueError("kv_cache must be [2, num_blocks, block_size, num_kv_heads, head_size]")
    return nb, b, hkv, d


def slot_mapping(block_tables: torch.Tensor, positions: torch.Tensor, block_size: int,
                 num_blocks: int, seq_ids: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int64 slot of each (sequence, position); -1 where nothing is written."""
    _need(block_tables, "block_tables", torch.int32, 2)
    dev = block_tables.device
    _need(positions, "positions", torch.int32, 1, dev)
    T = positions.shape[0]
    if seq_ids is not None:
        _need(seq_ids, "seq_ids", torch.int32, 1, dev)
        if seq_ids.shape[0] != T:
            raise ValueError("seq_ids and positions differ in length")
    elif T > block_tables.shape[0]:
        raise ValueError("without seq_ids, token i belongs to sequence i")
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, 1, dev)
    rc = lib.paged_kv_slot_mapping(out.data_ptr(), block_tables.data_ptr(), block_tables.shape[1],
                                   seq_ids.data_ptr() if seq_ids is not None else None,
                                   positions.data_ptr(), T, block_tables.shape[0], block_size,
                                   num_blocks, _stream(block_tables))
    check(rc, "paged_kv_slot_mapping")
    return out


def write(key: torch.Tensor, value: torch.Tensor, kv_cache: torch.Tensor,
          slot_mapping: torch.Tensor) -> None:
    """Store key[t] / value[t] ([T, Hkv, D]) at slot_mapping[t] of the cache."""
    nb, b, hkv, d = _cache_dims(kv_cache)
    dev = kv_cache.device
    for name, t in (("key", key), ("value", value)):
        _need(t, name, kv_cache.dtype, 3, dev)
        if tuple(t.shape[1:]) != (hkv, d):
            raise ValueError(f"{name} must be [T, {hkv}, {d}]")
    _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    T = key.shape[0]
    if value.shape[0] != T or slot_mapping.shape[0] != T:
        raise ValueError("key, value and slot_mapping differ in length")
    rc = lib.paged_kv_write(key.data_ptr(), value.data_ptr(), kv_cache.data_ptr(),
                            slot_mapping.data_ptr(), T, nb, b, hkv, d, _dt(kv_cache),
                            _stream(kv_cache))
    check(rc, "paged_kv_write")


def write_positions(key: torch.Tensor, value: torch.Tensor, kv_cache: torch.Tensor,
                    block_tables: torch.Tensor, positions: torch.Tensor,
                    seq_ids: Optional[torch.Tensor] = None,
                    slot_mapping: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """Store key[t] / value[t] at the slot of (seq_ids[t] or t, positions[t])
    found through the block tables, in one launch; fills ``slot_mapping``
    (int64 [T]) with the slots if given and returns it."""
    nb, b, hkv, d = _cache_dims(kv_cache)
    dev = kv_cache.device
    for name, t in (("key", key), ("value", value)):
        _need(t, name, kv_cache.dtype, 3, dev)
        if tuple(t.shape[1:]) != (hkv, d):
            raise ValueError(f"{name} must be [T, {hkv}, {d}]")
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(positions, "positions", torch.int32, 1, dev)
    T = key.shape[0]
    if value.shape[0] != T or positions.shape[0] != T:
        raise ValueError("key, value and positions differ in length")
    if seq_ids is not None:
        _need(seq_ids, "seq_ids", torch.int32, 1, dev)
        if seq_ids.shape[0] != T:
            raise ValueError("seq_ids and positions differ in length")
    elif T > block_tables.shape[0]:
        raise ValueError("without seq_ids, token i belongs to sequence i")
    if slot_mapping is not None:
        _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
        if slot_mapping.shape[0] != T:
            raise ValueError("slot_mapping must have one entry per token")
    rc = lib.paged_kv_write_positions(
        key.data_ptr(), value.data_ptr(), kv_cache.data_ptr(), block_tables.data_ptr(),
        block_tables.shape[1], seq_ids.data_ptr() if seq_ids is not None else None,
        positions.data_ptr(), slot_mapping.data_ptr() if slot_mapping is not None else None, T,
        block_tables.shape[0], nb, b, hkv, d, _dt(kv_cache), _stream(kv_cache))
    check(rc, "paged_kv_write_positions")
    return slot_mapping


def gather(kv_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
           max_context_len: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """K and V of every sequence in logical order: two [S, max_len, Hkv, D] tensors."""
    nb, b, hkv, d = _cache_dims(kv_cache)
    dev = kv_cache.device
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    S = context_lens.shape[0]
    if block_tables.shape[0] != S:
        raise ValueError("block_tables and context_lens differ in length")
    k = torch.empty((S, max_context_len, hkv, d), dtype=kv_cache.dtype, device=dev)
    v = torch.empty_like(k)
    rc = lib.paged_kv_gather(k.data_ptr(), v.data_ptr(), kv_cache.data_ptr(),
                             block_tables.data_ptr(), block_tables.shape[1],
                             context_lens.data_ptr(), S, hkv, d, b, nb, max_context_len,
                             _dt(kv_cache), _stream(kv_cache))
    check(rc, "paged_kv_gather")
    return k, v


def _pool_dims(t: torch.Tensor, name: str):
    """[2, nb, b, hkv, d] pool on a GPU or in pinned host memory."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be on a GPU or in pinned host memory")
    if not t.is_contiguous() or t.dim() != 5 or t.shape[0] != 2:
        raise ValueError(f"{name} must be a contiguous [2, num_blocks, block_size, "
                         "num_kv_heads, head_size] tensor")
    return tuple(t.shape[1:])


def copy_blocks(dst_cache: torch.Tensor, src_cache: torch.Tensor, src_blocks, dst_blocks) -> None:
    """dst_cache[:, dst_blocks[i]] = src_cache[:, src_blocks[i]] (keys and values).

    Copy-on-write copies (one pool) and swaps (a GPU pool and a pinned host
    pool of the same block geometry).  Block id lists may be int32 tensors on
    the GPU or Python sequences; the copy runs on the current stream of the
    GPU pool's device."""
    dnb, db, dh, dd = _pool_dims(dst_cache, "dst_cache")
    snb, sb, sh, sd = _pool_dims(src_cache, "src_cache")
    if (db, dh, dd) != (sb, sh, sd) or dst_cache.dtype != src_cache.dtype:
        raise ValueError("pools differ in block geometry or element type")
    gpu = dst_cache if dst_cache.is_cuda else src_cache
    if not gpu.is_cuda:
        raise ValueError("one pool must be on a GPU")
    ids = []
    for name, b in (("src_blocks", src_blocks), ("dst_blocks", dst_blocks)):
        if not isinstance(b, torch.Tensor):
            b = torch.tensor(list(b), dtype=torch.int32).to(gpu.device)
        _need(b, name, torch.int32, 1, gpu.device)
        ids.append(b)
    if ids[0].shape[0] != ids[1].shape[0]:
        raise ValueError("src_blocks and dst_blocks differ in length")
    rc = lib.paged_kv_copy_blocks(dst_cache.data_ptr(), dnb, src_cache.data_ptr(), snb,
                                  ids[0].data_ptr(), ids[1].data_ptr(), ids[0].shape[0],
                                  db, dh, dd, _dt(gpu), _stream(gpu))
    check(rc, "paged_kv_copy_blocks")


def partition_size(num_seqs, num_q_heads, num_kv_heads, head_size, block_size, max_context_len,
                   requested: int = 0, dtype: torch.dtype = torch.bfloat16) -> int:
    p = lib.paged_attention_partition_size(num_seqs, num_q_heads, num_kv_heads, head_size,
                                           block_size, max_context_len, requested, _DTYPES[dtype])
    if p < 0:
        raise PagedKVError(lib.pkv_last_error().decode())
    return p


def workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size, block_size, max_context_len,
                    requested: int = 0, dtype: torch.dtype = torch.bfloat16) -> int:
    return int(lib.paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size,
                                                   block_size, max_context_len, requested,
                                                   _DTYPES[dtype]))


def _decode_args(query, kv_cache, block_tables, context_lens, scale, max_context_len,
                 partition, out, out_dtype, workspace, shared_blocks=False):
    nb, b, hkv, d = _cache_dims(kv_cache)
    dev = kv_cache.device
    _need(query, "query", kv_cache.dtype, 3, dev)
    S, hq, dq = query.shape
    if dq != d:
        raise ValueError("query head_size differs from the cache's")
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("query, block_tables and context_lens differ in batch size")
    if out is None:
        out = torch.empty((S, hq, d), dtype=out_dtype, device=dev)
    _need(out, "out", None, 3, dev)
    if tuple(out.shape) != (S, hq, d):
        raise ValueError("out must be [S, Hq, D]")
    need = workspace_bytes(S, hq, hkv, d, b, max_context_len, partition, kv_cache.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    args = (out.data_ptr(), _dt(out), query.data_ptr(), kv_cache.data_ptr(),
            block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(), S, hq, hkv,
            d, b, nb, float(scale), int(max_context_len), int(partition), workspace.data_ptr(),
            workspace.numel(), _dt(kv_cache), PKV_ATTN_CACHED_KV if shared_blocks else 0,
            _stream(kv_cache))
    return out, args


def attention_decode(query: torch.Tensor, kv_cache: torch.Tensor, block_tables: torch.Tensor,
                     context_lens: torch.Tensor, scale: float, max_context_len: int,
                     partition_size: int = 0, out: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.float32,
                     workspace: Optional[torch.Tensor] = None,
                     shared_blocks: bool = False) -> torch.Tensor:
    """Paged decode attention; returns ``out`` [S, Hq, D].

    ``shared_blocks``: some physical blocks are referenced by several sequences
    of the batch; K/V are then read through the caches (PKV_ATTN_CACHED_KV).
    """
    out, args = _decode_args(query, kv_cache, block_tables, context_lens, scale, max_context_len,
                             partition_size, out, out_dtype, workspace, shared_blocks)
    check(lib.paged_attention_decode(*args), "paged_attention_decode")
    return out


def _split_call_buffers(n) -> None:
    """The two launches of a split call communicate through ``out`` and
    ``workspace``: both must be the caller's, the same for both calls."""
    if n[7] is None:
        raise ValueError("split decode calls need out= (the same tensor for both calls)")
    if n[9] is None:
        raise ValueError("split decode calls need workspace= (the same tensor for both calls)")


def attention_partitions(*a, **k) -> torch.Tensor:
    """First launch of attention_decode (attention pass); same arguments, and
    ``out`` and ``workspace`` must be given (the merge reads them)."""
    n = _norm(*a, **k)
    _split_call_buffers(n)
    out, args = _decode_args(*n)
    check(lib.paged_attention_partitions(*args), "paged_attention_partitions")
    return out


def attention_merge(*a, **k) -> torch.Tensor:
    """Second launch of attention_decode (log-sum-exp merge); same arguments,
    including the ``out`` and ``workspace`` the attention pass wrote."""
    n = _norm(*a, **k)
    _split_call_buffers(n)
    out, args = _decode_args(*n)
    check(lib.paged_attention_merge(*args), "paged_attention_merge")
    return out


def _append_args(key, value, query, kv_cache, args):
    """Decode arguments with the new tokens' key and value inserted."""
    shape = (query.shape[0], kv_cache.shape[3], kv_cache.shape[4])
    for t, name in ((key, "key"), (value, "value")):
        _need(t, name, kv_cache.dtype, 3, kv_cache.device)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be [S, Hkv, D] = {list(shape)}")
    return args[:3] + (key.data_ptr(), value.data_ptr()) + args[3:]


def attention_decode_append(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                            kv_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, scale: float, max_context_len: int,
                            partition_size: int = 0, out: Optional[torch.Tensor] = None,
                            out_dtype: torch.dtype = torch.float32,
                            workspace: Optional[torch.Tensor] = None,
                            shared_blocks: bool = False) -> torch.Tensor:
    """A decode step in one call: sequence s's new ``key[s]``/``value[s]``
    ([S, Hkv, D]) go to position ``context_lens[s] - 1`` of its blocks, then
    its query attends over all its tokens.  Returns ``out`` [S, Hq, D]."""
    out, args = _decode_args(query, kv_cache, block_tables, context_lens, scale, max_context_len,
                             partition_size, out, out_dtype, workspace, shared_blocks)
    check(lib.paged_attention_decode_append(*_append_args(key, value, query, kv_cache, args)),
          "paged_attention_decode_append")
    return out


def attention_append_partitions(query, key, value, *a, **k) -> torch.Tensor:
    """First launch of attention_decode_append (write + attention pass); follow it
    with attention_merge given the same decode arguments (``out`` and
    ``workspace`` included)."""
    n = _norm(query, *a, **k)
    _split_call_buffers(n)
    out, args = _decode_args(*n)
    check(lib.paged_attention_append_partitions(*_append_args(key, value, query, n[1], args)),
          "paged_attention_append_partitions")
    return out


def attention_prefill(query: torch.Tensor, kv_cache: torch.Tensor, block_tables: torch.Tensor,
                      context_lens: torch.Tensor, query_start: torch.Tensor, scale: float,
                      max_query_len: int, out_dtype=torch.float32,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal attention of each sequence's chunk of query rows
    (``query[query_start[s]:query_start[s+1]]``, the last tokens of sequence
    ``s``, whose K/V is already cached) over its paged K/V.  ``[T, Hq, D]``.
    ``max_query_len``: the longest chunk (a host int, as the caller's
    scheduler knows it); a longer chunk gives NaN rows."""
    nb, b, hkv, d = _cache_dims(kv_cache)
    dev = kv_cache.device
    _need(query, "query", kv_cache.dtype, 3, dev)
    T, hq, dq = query.shape
    if dq != d:
        raise ValueError(f"query head size {dq} differs from the cache's {d}")
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    _need(query_start, "query_start", torch.int32, 1, dev)
    S = context_lens.shape[0]
    if block_tables.shape[0] != S or query_start.shape[0] != S + 1:
        raise ValueError("block_tables, context_lens and query_start disagree on the batch")
    if out is None:
        out = torch.empty((T, hq, d), dtype=out_dtype, device=dev)
    _need(out, "out", None, 3, dev)
    if tuple(out.shape) != (T, hq, d) or out.dtype not in _DTYPES:
        raise ValueError("out must be a float32 or bfloat16 [T, Hq, D] tensor")
    rc = lib.paged_attention_prefill(out.data_ptr(), _dt(out), query.data_ptr(),
                                     query_start.data_ptr(), T, max_query_len, kv_cache.data_ptr(),
                                     block_tables.data_ptr(), block_tables.shape[1],
                                     context_lens.data_ptr(), S, hq, hkv, d, b, nb, float(scale),
                                     _dt(kv_cache), _stream(kv_cache))
    check(rc, "paged_attention_prefill")
    return out


def prefix_groups(block_tables, context_lens, block_size: int, min_prefix_len: int = 0):
    """Groups of consecutive sequences sharing their first blocks (host
    arrays; ``paged_attention_prefix_groups``).  Returns ``(group_starts
    [G + 1], prefix_lens [G], max_prefix_len)`` as int32 numpy arrays and an
    int."""
    import numpy as np
    tables = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    S = lens.shape[0]
    if tables.ndim != 2 or tables.shape[0] != S:
        raise ValueError("block_tables must be [S, width] for S context lengths")
    starts = np.zeros(S + 1, dtype=np.int32)
    plens = np.zeros(max(S, 1), dtype=np.int32)
    ng, mp = ctypes.c_int(0), ctypes.c_int(0)
    rc = lib.paged_attention_prefix_groups(tables.ctypes.data, tables.shape[1], lens.ctypes.data,
                                           S, int(block_size), int(min_prefix_len),
                                           starts.ctypes.data, plens.ctypes.data,
                                           ctypes.byref(ng), ctypes.byref(mp))
    check(rc, "paged_attention_prefix_groups")
    return starts[:ng.value + 1].copy(), plens[:ng.value].copy(), mp.value


def shared_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size, block_size, num_groups,
                           max_context_len, max_prefix_len, requested: int = 0) -> int:
    return int(lib.paged_attention_shared_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_size, block_size, num_groups, max_context_len,
        max_prefix_len, requested))


def shared_plan_bytes(num_seqs, num_q_heads, num_kv_heads, block_size, num_groups,
                      max_context_len, max_prefix_len, requested: int = 0) -> int:
    return int(lib.paged_attention_shared_plan_bytes(
        num_seqs, num_q_heads, num_kv_heads, block_size, num_groups, max_context_len,
        max_prefix_len, requested))


def make_shared_plan(block_tables: torch.Tensor, context_lens: torch.Tensor,
                     group_starts: torch.Tensor, prefix_lens: torch.Tensor, num_q_heads: int,
                     num_kv_heads: int, block_size: int, max_context_len: int,
                     max_prefix_len: int, partition_size: int = 0,
                     plan: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The work list of the shared-prefix decode for these tables, lengths and
    groups (``paged_attention_shared_plan``), to pass as ``plan`` to every
    :func:`attention_decode_shared` call over them (e.g. each layer of a
    decode step).  Returns ``plan``, a uint8 device tensor."""
    dev = block_tables.device
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    _need(group_starts, "group_starts", torch.int32, 1, dev)
    _need(prefix_lens, "prefix_lens", torch.int32, 1, dev)
    S, ng = block_tables.shape[0], prefix_lens.shape[0]
    if context_lens.shape[0] != S or group_starts.shape[0] != ng + 1:
        raise ValueError("block_tables, context_lens and the groups disagree in size")
    need = shared_plan_bytes(S, num_q_heads, num_kv_heads, block_size, ng, max_context_len,
                             max_prefix_len, partition_size)
    if plan is None:
        plan = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(plan, "plan", torch.uint8, 1, dev)
    rc = lib.paged_attention_shared_plan(
        plan.data_ptr(), plan.numel(), block_tables.data_ptr(), block_tables.shape[1],
        context_lens.data_ptr(), group_starts.data_ptr(), prefix_lens.data_ptr(), ng, S,
        num_q_heads, num_kv_heads, block_size, int(max_context_len), int(max_prefix_len),
        int(partition_size), _stream(block_tables))
    check(rc, "paged_attention_shared_plan")
    return plan


def attention_decode_shared(query: torch.Tensor, kv_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, group_starts: torch.Tensor,
                            prefix_lens: torch.Tensor, scale: float, max_context_len: int,
                            max_prefix_len: int, partition_size: int = 0,
                            out: Optional[torch.Tensor] = None,
                            out_dtype: torch.dtype = torch.float32,
                            workspace: Optional[torch.Tensor] = None,
                            cached_kv: bool = False,
                            plan: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged decode attention for groups of sequences sharing their first
    blocks (``paged_attention_decode_shared``): each group's prefix is read
    once for all its members.  ``group_starts`` [G + 1] and ``prefix_lens``
    [G] are int32 device tensors (see :func:`prefix_groups`).  With ``plan``
    (from :func:`make_shared_plan` over the same tables, lengths and groups)
    the work list is read from it (``paged_attention_decode_shared_planned``).
    Returns ``out``."""
    nb, b, hkv, d = _cache_dims(kv_cache)
    dev = kv_cache.device
    _need(query, "query", kv_cache.dtype, 3, dev)
    S, hq, dq = query.shape
    if dq != d:
        raise ValueError("query head_size differs from the cache's")
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    _need(group_starts, "group_starts", torch.int32, 1, dev)
    _need(prefix_lens, "prefix_lens", torch.int32, 1, dev)
    ng = prefix_lens.shape[0]
    if group_starts.shape[0] != ng + 1:
        raise ValueError("group_starts must have one more entry than prefix_lens")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("query, block_tables and context_lens differ in batch size")
    if out is None:
        out = torch.empty((S, hq, d), dtype=out_dtype, device=dev)
    _need(out, "out", None, 3, dev)
    if tuple(out.shape) != (S, hq, d):
        raise ValueError("out must be [S, Hq, D]")
    need = shared_workspace_bytes(S, hq, hkv, d, b, ng, max_context_len, max_prefix_len,
                                  partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    args = (out.data_ptr(), _dt(out), query.data_ptr(), kv_cache.data_ptr(),
            block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(),
            group_starts.data_ptr(), prefix_lens.data_ptr(), ng, S, hq, hkv, d, b, nb,
            float(scale), int(max_context_len), int(max_prefix_len), int(partition_size),
            workspace.data_ptr(), workspace.numel(), _dt(kv_cache),
            PKV_ATTN_CACHED_KV if cached_kv else 0)
    if plan is None:
        rc = lib.paged_attention_decode_shared(*args, _stream(kv_cache))
        check(rc, "paged_attention_decode_shared")
    else:
        _need(plan, "plan", torch.uint8, 1, dev)
        rc = lib.paged_attention_decode_shared_planned(*args, plan.data_ptr(), plan.numel(),
                                                       _stream(kv_cache))
        check(rc, "paged_attention_decode_shared_planned")
    return out


def _norm(query, kv_cache, block_tables, context_lens, scale, max_context_len,
          partition_size=0, out=None, out_dtype=torch.float32, workspace=None,
          shared_blocks=False):
    return (query, kv_cache, block_tables, context_lens, scale, max_context_len, partition_size,
            out, out_dtype, workspace, shared_blocks)
