"""Plain reference of the KV block manager: a ref-counted pool of physical
blocks with a free queue, sequences whose block tables map logical to
physical blocks, fork and copy-on-write, a prefix cache of full blocks keyed
by chain hashes, and swapping a group of sequences to a CPU pool and back.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is modelled, and from where:

* Every physical block has a reference count; a block shared by several
  logical blocks (forked samples) counts each of them [review, "요청 완료 후
  메모리 관리" (the two samples sharing blocks 7 and 1, counts 2)].
* Fork shares all of the parent's blocks and raises their counts; nothing is
  copied [explainer, section 3, the fork sketch].
* Before a token is written into a block whose count is above 1, the writer
  takes a fresh block, the old block's content is copied into it and the old
  count drops by one; a writer that finds count 1 writes in place [review,
  "생성 단계에서의 Copy-on-Write"; explainer, section 3, the copy-on-write
  sketch].  Only the block being written is copied [review, "메모리 복사
  오버헤드의 최적화"].
* Blocks fill left to right; a new block is taken only when the last one is
  full [review, "물리적 블록 할당"; walkthrough, the overall allocation flow].
  A prompt of n tokens takes ceil(n / B) blocks [walkthrough, "ブロック割当の
  ロジック": 10 tokens at B = 16 take 1 block].
* Free blocks wait in a queue; allocation takes them from its head; freeing a
  request returns its blocks -- those whose count reaches zero -- to the tail,
  last block first [walkthrough, "プレイフィックスキャッシュの詳細", times 4
  and 5 of the timeline, and "BlockPoolの生成過程"].
* A full block gets a chain hash, hash_i = H(hash_{i-1}, tokens of block i),
  and is registered in the cache; partial blocks get none [walkthrough,
  "プレイフィックスキャッシュの詳細"].  H is SHA-256 as in the timeline the page
  follows; the input is the previous hash (32 zero bytes before block 0)
  followed by the block's token ids as little-endian int32 (reading: the pages
  do not fix an encoding).
* A new request's prefix hits are the cached blocks of its leading full
  blocks, up to (n - 1) // B of them, stopping at the first miss; a hit block
  still in the free queue leaves it; the rest is allocated from the queue,
  and a cached block taken from the queue loses its cache entry (eviction on
  reuse) [walkthrough, "プレイフィックスキャッシュの詳細", find_longest_cache_hit
  and time 6].
* Running out of blocks refuses the request and changes nothing; a group of
  sequences sharing blocks is swapped out to a CPU pool, and back in, all or
  nothing; the CPU pool has its own allocator and a bounded number of blocks
  [review, "All-or-Nothing Eviction" and "스와핑(Swapping)"; walkthrough,
  "ブロックアロケーションの基本概念", the preemption paragraph].
"""
from __future__ import annotations

import hashlib
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

NONE_HASH = bytes(32)


class OutOfBlocks(Exception):
    """The pool cannot satisfy the request; no state was changed."""


def block_hash(parent: bytes, tokens: Sequence[int]) -> bytes:
    """Chain hash of one full block [walkthrough, "プレイフィックスキャッシュの詳細"]."""
    return hashlib.sha256(bytes(parent) + np.asarray(tokens, dtype="<i4").tobytes()).digest()


class _Seq:
    def __init__(self):
        self.table: List[int] = []       # physical block of each logical block
        self.tokens: List[int] = []      # token ids so far
        self.hashes: List[bytes] = []    # chain hash of each full block so far
        self.swapped = False             # table holds CPU blocks


class RefBlockManager:
    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = True,
                 num_cpu_blocks: int = 0, free_order: Optional[Sequence[int]] = None):
        self.N = num_blocks
        self.B = block_size
        self.prefix_caching = prefix_caching
        self.ref = [0] * num_blocks
        self.hash_of: List[Optional[bytes]] = [None] * num_blocks
        self.cache: Dict[bytes, int] = {}
        self.free: List[int] = list(range(num_blocks)) if free_order is None else list(free_order)
        assert sorted(self.free) == list(range(num_blocks))
        self.cpu_free: List[int] = list(range(num_cpu_blocks))
        self.cpu_ref = [0] * num_cpu_blocks
        self.seqs: Dict[int, _Seq] = {}

    # ------------------------------------------------------------ pool
    def _take(self) -> int:
        b = self.free.pop(0)
        h = self.hash_of[b]
        if h is not None:  # eviction on reuse
            if self.cache.get(h) == b:
                del self.cache[h]
            self.hash_of[b] = None
        self.ref[b] = 1
        return b

    def _touch(self, b: int) -> None:
        if self.ref[b] == 0:
            self.free.remove(b)
        self.ref[b] += 1

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def _cache_full(self, s: _Seq) -> None:
        while len(s.hashes) < len(s.tokens) // self.B:
            i = len(s.hashes)
            parent = s.hashes[-1] if s.hashes else NONE_HASH
            h = block_hash(parent, s.tokens[i * self.B:(i + 1) * self.B])
            s.hashes.append(h)
            if self.prefix_caching and not s.swapped:
                b = s.table[i]
                if h not in self.cache:
                    self.cache[h] = b
                if self.hash_of[b] is None:
                    self.hash_of[b] = h

    def _seq(self, sid: int) -> _Seq:
        if sid not in self.seqs:
            raise KeyError(sid)
        return self.seqs[sid]

    # ------------------------------------------------------------ requests
    def allocate(self, sid: int, tokens: Sequence[int]) -> int:
        """Admit a request of len(tokens) tokens; returns the number of
        leading tokens found in the prefix cache."""
        if sid in self.seqs:
            raise KeyError(sid)
        n = len(tokens)
        need = -(-n // self.B)
        hits: List[int] = []
        if self.prefix_caching:
            parent = NONE_HASH
            for i in range((n - 1) // self.B if n > 0 else 0):
                h = block_hash(parent, tokens[i * self.B:(i + 1) * self.B])
                b = self.cache.get(h)
                if b is None:
                    break
                hits.append(b)
                parent = h
        in_queue = sum(1 for b in hits if self.ref[b] == 0)
        if len(self.free) - in_queue < need - len(hits):
            raise OutOfBlocks()
        s = _Seq()
        for b in hits:
            self._touch(b)
        s.table = hits + [self._take() for _ in range(need - len(hits))]
        s.tokens = list(tokens)
        self.seqs[sid] = s
        self._cache_full(s)
        return len(hits) * self.B

    def append(self, sid: int, tokens: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Decode: write len(tokens) new tokens.  Returns their slots and the
        (source, destination) block copies copy-on-write needs first."""
        s = self._seq(sid)
        if s.swapped:
            raise KeyError(sid)
        # the blocks this needs -- one per new logical block, one per shared
        # block written -- so as to refuse before changing anything
        if tokens:
            first, last = len(s.tokens) // self.B, (len(s.tokens) + len(tokens) - 1) // self.B
            need = sum(1 for lb in range(first, last + 1)
                       if lb >= len(s.table) or self.ref[s.table[lb]] > 1)
            if need > len(self.free):
                raise OutOfBlocks()
        slots, copies = [], []
        for t in tokens:
            p = len(s.tokens)
            lb = p // self.B
            if lb == len(s.table):
                s.table.append(self._take())
            elif self.ref[s.table[lb]] > 1:
                old = s.table[lb]
                nb = self._take()
                copies.append((old, nb))
                self.ref[old] -= 1  # still held by the other sharers
                s.table[lb] = nb
            slots.append(s.table[lb] * self.B + p % self.B)
            s.tokens.append(int(t))
            self._cache_full(s)
        return slots, copies

    def fork(self, parent: int, child: int) -> None:
        s = self._seq(parent)
        if child in self.seqs or s.swapped:
            raise KeyError(child)
        c = _Seq()
        c.table, c.tokens, c.hashes = list(s.table), list(s.tokens), list(s.hashes)
        for b in c.table:
            self.ref[b] += 1
        self.seqs[child] = c

    def free_seq(self, sid: int) -> None:
        s = self._seq(sid)
        if s.swapped:
            for b in reversed(s.table):
                self._cpu_release(b)
        else:
            for b in reversed(s.table):
                self._release(b)
        del self.seqs[sid]

    # ------------------------------------------------------------ swapping
    def _cpu_release(self, b: int) -> None:
        self.cpu_ref[b] -= 1
        if self.cpu_ref[b] == 0:
            self.cpu_free.append(b)

    def swap_out(self, sids: Sequence[int]) -> List[Tuple[int, int]]:
        """Move every block of the group to the CPU pool (all or nothing).
        Returns (GPU block, CPU block) copies, in first-use order."""
        group = [self._seq(i) for i in sids]
        if any(s.swapped for s in group):
            raise KeyError("already swapped")
        blocks: List[int] = []
        uses: Dict[int, int] = {}
        for s in group:
            for b in s.table:
                if b not in uses:
                    blocks.append(b)
                uses[b] = uses.get(b, 0) + 1
        if any(self.ref[b] != uses[b] for b in blocks):
            raise KeyError("blocks shared outside the group")
        if len(blocks) > len(self.cpu_free):
            raise OutOfBlocks()
        to_cpu = {b: self.cpu_free.pop(0) for b in blocks}
        for b in blocks:
            self.cpu_ref[to_cpu[b]] = uses[b]
        for s in group:
            s.table = [to_cpu[b] for b in s.table]
            s.swapped = True
        for b in reversed(blocks):
            h = self.hash_of[b]
            if h is not None:
                if self.cache.get(h) == b:
                    del self.cache[h]
                self.hash_of[b] = None
            self.ref[b] = 0
            self.free.append(b)
        return [(b, to_cpu[b]) for b in blocks]

    def swap_in(self, sids: Sequence[int]) -> List[Tuple[int, int]]:
        """Bring a swapped group back (all or nothing).  Returns (CPU block,
        GPU block) copies, in first-use order."""
        group = [self._seq(i) for i in sids]
        if not all(s.swapped for s in group):
            raise KeyError("not swapped")
        blocks: List[int] = []
        uses: Dict[int, int] = {}
        for s in group:
            for b in s.table:
                if b not in uses:
                    blocks.append(b)
                uses[b] = uses.get(b, 0) + 1
        if any(self.cpu_ref[b] != uses[b] for b in blocks):
            raise KeyError("blocks shared outside the group")
        if len(blocks) > len(self.free):
            raise OutOfBlocks()
        to_gpu = {b: self._take() for b in blocks}
        for b in blocks:
            self.ref[to_gpu[b]] = self.cpu_ref[b]
        for s in group:
            s.table = [to_gpu[b] for b in s.table]
            s.swapped = False
        for b in reversed(blocks):
            self.cpu_ref[b] = 0
            self.cpu_free.append(b)
        for s in group:
            # full blocks are cached again under their (unchanged) hashes
            if self.prefix_caching:
                for i, h in enumerate(s.hashes):
                    b = s.table[i]
                    if h not in self.cache:
                        self.cache[h] = b
                    if self.hash_of[b] is None:
                        self.hash_of[b] = h
        return [(b, to_gpu[b]) for b in blocks]

    # ------------------------------------------------------------ views
    def table(self, sid: int) -> List[int]:
        return list(self._seq(sid).table)

    def num_tokens(self, sid: int) -> int:
        return len(self._seq(sid).tokens)

    def slots(self, sid: int, begin: int, end: int) -> List[int]:
        s = self._seq(sid)
        return [s.table[p // self.B] * self.B + p % self.B for p in range(begin, end)]


def copy_blocks_ref(kv: np.ndarray, pairs: Sequence[Tuple[int, int]],
                    dst: Optional[np.ndarray] = None) -> np.ndarray:
    """Copy whole blocks (keys and values) ``src -> dst`` between pools laid
    out as ``[2, NB, B, Hkv, D]`` -- the copy-on-write copy [review,
    "생성 단계에서의 Copy-on-Write": block 1's content copied into block 3] and
    the swap of a block between the GPU and CPU pools.  Copies are
    independent: no destination is also a source."""
    out = kv if dst is None else dst
    for s, d in pairs:
        out[:, d] = kv[:, s]
    return out
