"""Python handle on the library's host block manager (``pkv_bm_*`` in
include/paged_kv.h): argument marshalling only; the allocator itself is the
C++ in ``csrc/block_manager.cpp``."""
from __future__ import annotations

import ctypes
from typing import List, Sequence, Tuple

import numpy as np

from ._lib import PKV_ERR_NO_BLOCKS, PagedKVError, check, lib


class NoFreeBlocks(PagedKVError):
    """The pool could not satisfy the request; nothing was changed."""


def _call(rc: int, what: str) -> int:
    if rc == PKV_ERR_NO_BLOCKS:
        raise NoFreeBlocks(f"{what}: {lib.pkv_last_error().decode(errors='replace')}")
    if rc < 0:
        check(rc, what)
    return rc


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class BlockManager:
    """Block tables, slots and copy lists for one pool of ``num_blocks``
    blocks of ``block_size`` tokens (see pkv_bm_* in include/paged_kv.h)."""

    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = True,
                 num_cpu_blocks: int = 0, free_order: Sequence[int] = None):
        self._h = lib.pkv_bm_create(num_blocks, block_size, int(prefix_caching), num_cpu_blocks)
        if not self._h:
            raise PagedKVError(lib.pkv_last_error().decode(errors="replace"))
        self.num_blocks, self.block_size = num_blocks, block_size
        if free_order is not None:
            order = _i32(free_order)
            _call(lib.pkv_bm_set_free_order(self._h, _ptr(order), len(order)), "set_free_order")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib.pkv_bm_destroy(h)
            self._h = None

    def allocate(self, seq: int, tokens: Sequence[int]) -> int:
        t = _i32(tokens)
        cached = ctypes.c_int(0)
        _call(lib.pkv_bm_allocate(self._h, seq, _ptr(t), len(t), ctypes.byref(cached)), "allocate")
        return cached.value

    def append(self, seq: int, tokens: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        t = _i32(tokens)
        n = len(t)
        slots = np.zeros(max(n, 1), dtype=np.int64)
        src, dst = np.zeros(max(n, 1), dtype=np.int32), np.zeros(max(n, 1), dtype=np.int32)
        nc = ctypes.c_int(0)
        _call(lib.pkv_bm_append(self._h, seq, _ptr(t), n, _ptr(slots), _ptr(src), _ptr(dst),
                                ctypes.byref(nc)), "append")
        return slots[:n].tolist(), list(zip(src[:nc.value].tolist(), dst[:nc.value].tolist()))

    def fork(self, parent: int, child: int) -> None:
        _call(lib.pkv_bm_fork(self._h, parent, child), "fork")

    def free(self, seq: int) -> None:
        _call(lib.pkv_bm_free(self._h, seq), "free")

    def _swap(self, fn, seqs: Sequence[int], what: str) -> List[Tuple[int, int]]:
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        cap = self.num_blocks
        a, b = np.zeros(cap, dtype=np.int32), np.zeros(cap, dtype=np.int32)
        nc = ctypes.c_int(0)
        _call(fn(self._h, _ptr(ids), len(ids), _ptr(a), _ptr(b), cap, ctypes.byref(nc)), what)
        return list(zip(a[:nc.value].tolist(), b[:nc.value].tolist()))

    def swap_out(self, seqs: Sequence[int]) -> List[Tuple[int, int]]:
        """(GPU block, CPU block) copies to make."""
        return self._swap(lib.pkv_bm_swap_out, seqs, "swap_out")

    def swap_in(self, seqs: Sequence[int]) -> List[Tuple[int, int]]:
        """(CPU block, GPU block) copies to make."""
        return self._swap(lib.pkv_bm_swap_in, seqs, "swap_in")

    def num_tokens(self, seq: int) -> int:
        return _call(lib.pkv_bm_num_tokens(self._h, seq), "num_tokens")

    def is_swapped(self, seq: int) -> bool:
        return bool(_call(lib.pkv_bm_is_swapped(self._h, seq), "is_swapped"))

    def table(self, seq: int) -> List[int]:
        n = _call(lib.pkv_bm_block_table(self._h, seq, None, 0), "block_table")
        out = np.zeros(max(n, 1), dtype=np.int32)
        _call(lib.pkv_bm_block_table(self._h, seq, _ptr(out), n), "block_table")
        return out[:n].tolist()

    def slots(self, seq: int, begin: int, end: int) -> List[int]:
        out = np.zeros(max(end - begin, 1), dtype=np.int64)
        _call(lib.pkv_bm_slots(self._h, seq, begin, end, _ptr(out)), "slots")
        return out[:end - begin].tolist()

    def batch_tables(self, seqs: Sequence[int], width: int) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        tables = np.zeros((len(ids), width), dtype=np.int32)
        lens = np.zeros(len(ids), dtype=np.int32)
        _call(lib.pkv_bm_batch_tables(self._h, _ptr(ids), len(ids), _ptr(tables), width, _ptr(lens)),
              "batch_tables")
        return tables, lens

    def ref_count(self, block: int) -> int:
        return _call(lib.pkv_bm_ref_count(self._h, block), "ref_count")

    def ref_counts(self) -> List[int]:
        return [self.ref_count(b) for b in range(self.num_blocks)]

    def num_free(self) -> int:
        return _call(lib.pkv_bm_num_free(self._h), "num_free")

    def free_queue(self) -> List[int]:
        out = np.zeros(self.num_blocks, dtype=np.int32)
        n = _call(lib.pkv_bm_free_queue(self._h, _ptr(out), self.num_blocks), "free_queue")
        return out[:n].tolist()

    def block_hash(self, block: int):
        out = np.zeros(32, dtype=np.uint8)
        has = _call(lib.pkv_bm_block_hash(self._h, block, _ptr(out)), "block_hash")
        return out.tobytes() if has else None

    def cached_blocks(self) -> List[int]:
        return [b for b in range(self.num_blocks) if _call(lib.pkv_bm_is_cached(self._h, b), "is_cached")]
