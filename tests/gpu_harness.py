"""Helpers for the GPU tests and the benchmark: put a workload on the device
and drive the library through its Python binding (hence its C ABI).

The device pool starts as all-NaN; the cached tokens are placed by the
library's own slot-mapping and write kernels, the same path a decode step
uses, so nothing the GPU reads is computed by the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import paged_kv_cache_81_amd as pkv
import workloads

NAN_BF16 = 0x7FC0


def to_torch(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def nan_pool_numpy(w: workloads.Workload) -> np.ndarray:
    shape = (2, w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
    if w.dtype == "bf16":
        return np.full(shape, NAN_BF16, dtype=np.uint16)
    return np.full(shape, np.nan, dtype=np.float32)


@dataclass
class DeviceStep:
    w: workloads.Workload
    kv: torch.Tensor
    query: torch.Tensor
    tables: torch.Tensor
    lens: torch.Tensor
    new_k: torch.Tensor
    new_v: torch.Tensor
    new_pos: torch.Tensor
    new_slots: torch.Tensor


def upload(w: workloads.Workload, device="cuda:0", fill=True, step=True) -> DeviceStep:
    """Device copies of a workload's inputs; the pool is NaN, then (``fill``)
    every cached token is written, then (``step``) each sequence's new token."""
    dev = torch.device(device)
    kv = to_torch(nan_pool_numpy(w), w.dtype, dev)
    tables = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    st = DeviceStep(
        w=w, kv=kv, query=to_torch(w.query, w.dtype, dev), tables=tables, lens=lens,
        new_k=to_torch(w.new_k, w.dtype, dev), new_v=to_torch(w.new_v, w.dtype, dev),
        new_pos=torch.from_numpy(w.new_pos).to(dev),
        new_slots=torch.empty(w.num_seqs, dtype=torch.int64, device=dev))
    if fill and w.cached_k.shape[0]:
        fill_cached(st)
    if step:
        run_write_step(st)
    return st


def fill_cached(st: DeviceStep, chunk_rows: int = 1 << 18) -> None:
    w = st.w
    dev = st.kv.device
    N = w.cached_k.shape[0]
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        seq = torch.from_numpy(w.cached_seq[r0:r1]).to(dev)
        pos = torch.from_numpy(w.cached_pos[r0:r1]).to(dev)
        slots = pkv.slot_mapping(st.tables, pos, w.block_size, w.num_blocks, seq_ids=seq)
        pkv.write(to_torch(w.cached_k[r0:r1], w.dtype, dev), to_torch(w.cached_v[r0:r1], w.dtype, dev),
                  st.kv, slots)


def run_write_step(st: DeviceStep) -> None:
    """The write half of a decode step: slot of each new token, then the write."""
    w = st.w
    pkv.slot_mapping(st.tables, st.new_pos, w.block_size, w.num_blocks, out=st.new_slots)
    pkv.write(st.new_k, st.new_v, st.kv, st.new_slots)


def attend(st: DeviceStep, partition_size=None, out_dtype=torch.float32,
           shared_blocks=None) -> torch.Tensor:
    """Decode attention over the device step; workloads that alias blocks
    across sequences read K/V through the caches unless told otherwise."""
    w = st.w
    P = w.partition_size if partition_size is None else partition_size
    shared = bool(w.meta.get("forks")) if shared_blocks is None else shared_blocks
    return pkv.attention_decode(st.query, st.kv, st.tables, st.lens, w.scale, w.max_context_len,
                                partition_size=P, out_dtype=out_dtype, shared_blocks=shared)


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per output row (last axis): max |got - ref| / max |ref|."""
    err = np.abs(got.astype(np.float64) - ref).max(axis=-1)
    mag = np.abs(ref).max(axis=-1)
    return err / np.maximum(mag, 1e-30)


def tolerance(w: workloads.Workload) -> float:
    return 2e-3 if w.dtype == "bf16" else 1e-5
