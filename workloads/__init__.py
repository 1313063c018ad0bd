"""Seeded synthetic inputs for one paged decode step.

This module draws random numbers and lays out the *inputs* of a decode step the
way a host-side block allocator would hand them to the GPU:

* per-sequence context lengths ``L_s`` (they count the token appended this
  step, which sits at position ``L_s - 1``);
* per-sequence block tables: row ``s`` lists the physical block ids that hold
  logical blocks 0, 1, ... of sequence ``s``; unused entries hold
  ``TABLE_PAD``;
* query vectors, the K/V of every token already cached before the step, and
  the K/V of the token each sequence appends this step.

It holds none of the method's arithmetic.  It never turns a position into a
slot, never reads a cache through a table and never computes attention: the
HIP path and the CPU oracle each do that on their own from what this module
returns.  Cached tokens are described by the pair (sequence, position) whose
slot they occupy; each side derives the slot itself.

Floating-point inputs are drawn as float32 N(0, 1).  For bf16 workloads they
are rounded to nearest-even bf16 and handed to both sides as the raw 16-bit
patterns (``numpy.uint16``), so both sides see identical values.

The five named workloads follow the shapes the pages' examples and the
project's benchmark plan use (an OPT-13B-shaped MHA layer, a Qwen2-0.5B-shaped
GQA layer, parallel sampling over a shared prompt, a long-context batch); no
model weights or datasets are involved.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

TABLE_PAD = np.int32(-2**31)  # value of block-table entries that hold no block

_ROW_CHUNK = 1 << 10  # rows per independently seeded chunk


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """Inputs of one decode step over one attention layer.

    Arrays hold float32 values for ``dtype == "f32"`` and bf16 bit patterns
    (uint16) for ``dtype == "bf16"``.
    """

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    scale: float
    partition_size: int              # 0 lets the library choose
    context_lens: np.ndarray         # int32 [S]
    block_tables: np.ndarray         # int32 [S, width]
    query: np.ndarray                # [S, Hq, D]
    cached_k: np.ndarray             # [N, Hkv, D]
    cached_v: np.ndarray             # [N, Hkv, D]
    cached_seq: np.ndarray           # int32 [N]: sequence whose table places the row
    cached_pos: np.ndarray           # int32 [N]: position of the row in that sequence
    new_k: np.ndarray                # [S, Hkv, D]: token appended this step
    new_v: np.ndarray                # [S, Hkv, D]
    new_pos: np.ndarray              # int32 [S]: its position, -1 if none is appended
    seq_rows: np.ndarray             # int64 [sum L]: logical token order, as row ids
    seq_rows_start: np.ndarray       # int64 [S + 1]: sequence s owns seq_rows[start[s]:start[s+1]]
    meta: Dict[str, object] = field(default_factory=dict)

    # Row ids in ``seq_rows`` index the concatenation (cached rows, new rows):
    # ids below N are cached rows, id N + s is the new token of sequence s.

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def table_width(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def logical_rows(self, s: int) -> np.ndarray:
        return self.seq_rows[self.seq_rows_start[s]:self.seq_rows_start[s + 1]]

    def logical_kv(self, s: int):
        """K and V of sequence ``s`` in position order, ``[L_s, Hkv, D]`` each."""
        rows = self.logical_rows(s)
        n = self.cached_k.shape[0]
        cached = rows < n
        k = np.empty((rows.shape[0],) + self.cached_k.shape[1:], dtype=self.cached_k.dtype)
        v = np.empty_like(k)
        k[cached] = self.cached_k[rows[cached]]
        v[cached] = self.cached_v[rows[cached]]
        k[~cached] = self.new_k[rows[~cached] - n]
        v[~cached] = self.new_v[rows[~cached] - n]
        return k, v


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) draws of ``shape`` in the workload's element representation.

    One 63-bit seed is taken from ``rng``; the array is then drawn in chunks of
    ``_ROW_CHUNK`` rows, chunk ``i`` from its own PCG64 stream seeded with
    (seed, i).  Chunks are independent, so they are drawn in parallel threads
    and the result does not depend on the number of threads.
    """
    seed = int(rng.integers(0, 2**63 - 1))
    rows = shape[0]
    inner = tuple(shape[1:])
    out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)

    def draw(i: int) -> None:
        r0 = i * _ROW_CHUNK
        r1 = min(rows, r0 + _ROW_CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, i])))
        x = g.standard_normal((r1 - r0,) + inner, dtype=np.float32)
        out[r0:r1] = x if dtype == "f32" else to_bf16_bits(x)

    nchunks = (rows + _ROW_CHUNK - 1) // _ROW_CHUNK
    if nchunks <= 1:
        for i in range(nchunks):
            draw(i)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1, nchunks)) as ex:
            list(ex.map(draw, range(nchunks)))
    return out


def normal(seed: int, shape, dtype: str = "bf16") -> np.ndarray:
    """Seeded N(0,1) array of ``shape`` (bf16 bit patterns or float32)."""
    return _normal(np.random.default_rng(seed), shape, dtype)


def _blocks_to_hold(lens: np.ndarray, block_size: int) -> np.ndarray:
    """Blocks an allocator reserves so that ``len`` tokens fit (ceiling division)."""
    return np.ceil(np.asarray(lens, dtype=np.float64) / block_size).astype(np.int64)


def _independent(name: str, rng: np.random.Generator, lens: Sequence[int], *, dtype: str,
                 num_q_heads: int, num_kv_heads: int, head_size: int, block_size: int,
                 num_blocks: Optional[int] = None, pool_factor: float = 1.25,
                 table_width: Optional[int] = None, partition_size: int = 0,
                 scale: Optional[float] = None) -> Workload:
    """Sequences that own all their blocks (no sharing).

    Draw order after the lengths: block permutation, query, cached K, cached V,
    new K, new V.
    """
    lens = np.asarray(lens, dtype=np.int64)
    S = lens.shape[0]
    Hkv, D, B = num_kv_heads, head_size, block_size
    nblk = _blocks_to_hold(lens, B)
    needed = int(nblk.sum())
    if num_blocks is None:
        num_blocks = max(1, int(np.ceil(pool_factor * needed)))
    if num_blocks < needed:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {needed}")
    width = int(table_width if table_width is not None else max(1, int(nblk.max()) if S else 1))
    if S and width < nblk.max():
        raise ValueError("table width too small")
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((S, width), TABLE_PAD, dtype=np.int32)
    off = 0
    for s in range(S):
        tables[s, :nblk[s]] = perm[off:off + nblk[s]]
        off += nblk[s]
    query = _normal(rng, (S, num_q_heads, D), dtype)
    ncached = np.maximum(lens - 1, 0)
    N = int(ncached.sum())
    cached_k = _normal(rng, (N, Hkv, D), dtype)
    cached_v = _normal(rng, (N, Hkv, D), dtype)
    new_k = _normal(rng, (S, Hkv, D), dtype)
    new_v = _normal(rng, (S, Hkv, D), dtype)
    cached_seq = np.repeat(np.arange(S, dtype=np.int32), ncached)
    starts = np.concatenate([[0], np.cumsum(ncached)]).astype(np.int64)
    cached_pos = (np.arange(N, dtype=np.int64) - np.repeat(starts[:-1], ncached)).astype(np.int32)
    new_pos = np.where(lens > 0, lens - 1, -1).astype(np.int32)
    rows: List[np.ndarray] = []
    for s in range(S):
        if lens[s] == 0:
            rows.append(np.zeros(0, dtype=np.int64))
            continue
        rows.append(np.concatenate([np.arange(starts[s], starts[s + 1], dtype=np.int64),
                                    np.array([N + s], dtype=np.int64)]))
    seq_rows_start = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    seq_rows = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return Workload(
        name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=Hkv, head_size=D,
        block_size=B, num_blocks=int(num_blocks),
        scale=float(scale if scale is not None else 1.0 / np.sqrt(D)),
        partition_size=partition_size, context_lens=lens.astype(np.int32), block_tables=tables,
        query=query, cached_k=cached_k, cached_v=cached_v, cached_seq=cached_seq,
        cached_pos=cached_pos, new_k=new_k, new_v=new_v, new_pos=new_pos, seq_rows=seq_rows,
        seq_rows_start=seq_rows_start)


def _shared_prefix(name: str, rng: np.random.Generator, *, num_prompts: int, prompt_len: int,
                   forks: int, max_private: int, dtype: str, num_q_heads: int,
                   num_kv_heads: int, head_size: int, block_size: int,
                   pool_factor: float = 1.25, partition_size: int = 0) -> Workload:
    """Parallel sampling: ``forks`` sequences per prompt alias the prompt's blocks.

    Each fork then owns ``n ~ U{0..max_private}`` private tokens in blocks of its
    own.  A fork with ``n == 0`` appends nothing this step (its last position
    lies in a shared block, which would need a copy-on-write first).  Sequence
    ``p * forks + f`` is fork ``f`` of prompt ``p``.
    """
    Hkv, D, B = num_kv_heads, head_size, block_size
    S = num_prompts * forks
    n_priv = rng.integers(0, max_private + 1, size=S).astype(np.int64)
    lens = prompt_len + n_priv
    prompt_blocks = int(_blocks_to_hold(np.array([prompt_len]), B)[0])
    if prompt_blocks * B != prompt_len:
        raise ValueError("shared prompts must fill whole blocks (no copy-on-write here)")
    priv_blocks = _blocks_to_hold(lens, B) - prompt_blocks
    needed = num_prompts * prompt_blocks + int(priv_blocks.sum())
    num_blocks = int(np.ceil(pool_factor * needed))
    width = int(prompt_blocks + priv_blocks.max())
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((S, width), TABLE_PAD, dtype=np.int32)
    off = 0
    for p in range(num_prompts):
        shared = perm[off:off + prompt_blocks]
        off += prompt_blocks
        for f in range(forks):
            s = p * forks + f
            tables[s, :prompt_blocks] = shared
            tables[s, prompt_blocks:prompt_blocks + priv_blocks[s]] = perm[off:off + priv_blocks[s]]
            off += priv_blocks[s]
    query = _normal(rng, (S, num_q_heads, D), dtype)
    # cached rows: each prompt once (placed through its first fork's table),
    # then every fork's private tokens that precede its new token
    n_cached_priv = np.maximum(n_priv - 1, 0)
    N = num_prompts * prompt_len + int(n_cached_priv.sum())
    cached_k = _normal(rng, (N, Hkv, D), dtype)
    cached_v = _normal(rng, (N, Hkv, D), dtype)
    new_k = _normal(rng, (S, Hkv, D), dtype)
    new_v = _normal(rng, (S, Hkv, D), dtype)
    cached_seq = np.empty(N, dtype=np.int32)
    cached_pos = np.empty(N, dtype=np.int32)
    prompt_row0 = np.arange(num_prompts, dtype=np.int64) * prompt_len
    for p in range(num_prompts):
        cached_seq[p * prompt_len:(p + 1) * prompt_len] = p * forks
        cached_pos[p * prompt_len:(p + 1) * prompt_len] = np.arange(prompt_len)
    r = num_prompts * prompt_len
    rows: List[np.ndarray] = []
    new_pos = np.full(S, -1, dtype=np.int32)
    for s in range(S):
        p = s // forks
        k = int(n_cached_priv[s])
        cached_seq[r:r + k] = s
        cached_pos[r:r + k] = prompt_len + np.arange(k)
        parts = [prompt_row0[p] + np.arange(prompt_len, dtype=np.int64),
                 np.arange(r, r + k, dtype=np.int64)]
        if n_priv[s] > 0:
            new_pos[s] = lens[s] - 1
            parts.append(np.array([N + s], dtype=np.int64))
        rows.append(np.concatenate(parts))
        r += k
    seq_rows_start = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return Workload(
        name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=Hkv, head_size=D,
        block_size=B, num_blocks=num_blocks, scale=float(1.0 / np.sqrt(D)),
        partition_size=partition_size, context_lens=lens.astype(np.int32), block_tables=tables,
        query=query, cached_k=cached_k, cached_v=cached_v, cached_seq=cached_seq,
        cached_pos=cached_pos, new_k=new_k, new_v=new_v, new_pos=new_pos,
        seq_rows=np.concatenate(rows), seq_rows_start=seq_rows_start,
        meta={"num_prompts": num_prompts, "forks": forks, "prompt_len": prompt_len})


# --------------------------------------------------------------------------
# the five named workloads

def tiny(seed: int = 81000) -> Workload:
    """4 sequences of {7, 33, 100, 250} tokens, MHA 4/4, D 64, B 16, fp32, pool 64."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _independent("tiny", rng, [7, 33, 100, 250], dtype="f32", num_q_heads=4,
                        num_kv_heads=4, head_size=64, block_size=16, num_blocks=64,
                        table_width=16, scale=1.0 / 8.0)


def opt13b_mha(seed: int = 81001, num_seqs: int = 64, lo: int = 256, hi: int = 2048,
               num_heads: int = 40, block_size: int = 16) -> Workload:
    """OPT-13B-shaped MHA layer: 40/40 heads, D 128, B 16, bf16, L ~ U[lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(lo, hi + 1, size=num_seqs)
    return _independent("opt13b_mha", rng, lens, dtype="bf16", num_q_heads=num_heads,
                        num_kv_heads=num_heads, head_size=128, block_size=block_size)


def qwen2_gqa(seed: int = 81002, num_seqs: int = 256, median: float = 512.0,
              sigma: float = 1.0, lo: int = 16, hi: int = 8192,
              block_size: int = 16) -> Workload:
    """Qwen2-0.5B-shaped GQA layer: 14/2 heads, D 64, B 16, bf16, log-normal lengths."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.clip(np.rint(np.exp(np.log(median) + sigma * rng.standard_normal(num_seqs))),
                   lo, hi).astype(np.int64)
    return _independent("qwen2_gqa", rng, lens, dtype="bf16", num_q_heads=14,
                        num_kv_heads=2, head_size=64, block_size=block_size)


def shared_prefix(seed: int = 81003, num_prompts: int = 32, prompt_len: int = 1024,
                  forks: int = 8, max_private: int = 256, *, num_q_heads: int = 32,
                  num_kv_heads: int = 8, head_size: int = 128, block_size: int = 16) -> Workload:
    """32 prompts of 1024 tokens, 8 forks each aliasing them, 0-256 private
    tokens (GQA 32/8, D 128, B 16, bf16; other head and block shapes for
    parity cases)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _shared_prefix("shared_prefix", rng, num_prompts=num_prompts,
                          prompt_len=prompt_len, forks=forks, max_private=max_private,
                          dtype="bf16", num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                          head_size=head_size, block_size=block_size)


def long_context(seed: int = 81004, num_seqs: int = 16, context_len: int = 32768,
                 partition_size: int = 0) -> Workload:
    """16 sequences of 32768 tokens, GQA 64/8, D 128, B 32, bf16, fully shuffled pool.

    The natural split is 64 partitions of 512 tokens per sequence
    (``partition_size=512``); by default the library chooses, which on this
    shape is the balanced stream schedule."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.full(num_seqs, context_len, dtype=np.int64)
    needed = int(_blocks_to_hold(lens, 32).sum())
    return _independent("long_context", rng, lens, dtype="bf16", num_q_heads=64,
                        num_kv_heads=8, head_size=128, block_size=32, num_blocks=needed,
                        partition_size=partition_size)


def custom(seed: int, lens: Sequence[int], *, dtype: str = "bf16", num_q_heads: int = 8,
           num_kv_heads: int = 2, head_size: int = 128, block_size: int = 16,
           num_blocks: Optional[int] = None, pool_factor: float = 1.25,
           table_width: Optional[int] = None, partition_size: int = 0,
           scale: Optional[float] = None, name: str = "custom") -> Workload:
    """Independent sequences of the given lengths (edge cases and small parity cases)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _independent(name, rng, lens, dtype=dtype, num_q_heads=num_q_heads,
                        num_kv_heads=num_kv_heads, head_size=head_size, block_size=block_size,
                        num_blocks=num_blocks, pool_factor=pool_factor, table_width=table_width,
                        partition_size=partition_size, scale=scale)


# --------------------------------------------------------------------------
# prefill (chunked) workloads

@dataclass
class PrefillWorkload:
    """Inputs of one prefill step: each sequence's chunk of ``chunk_lens[s]``
    query tokens ends its ``cache.context_lens[s]`` tokens, all of whose K/V
    (the cached prefix and the chunk's own) is written before attention.
    ``cache`` describes the pool, the tables and those K/V rows (its decode
    query is unused); ``query`` holds the chunks' rows, sequence ``s`` at
    ``query_start[s] .. query_start[s+1]-1``."""

    name: str
    cache: Workload
    chunk_lens: np.ndarray    # int32 [S]
    query_start: np.ndarray   # int32 [S + 1]
    query: np.ndarray         # [T, Hq, D]

    @property
    def num_tokens(self) -> int:
        return int(self.query_start[-1])

    @property
    def max_query_len(self) -> int:
        return int(self.chunk_lens.max()) if self.chunk_lens.size else 0

    def flops(self) -> int:
        """4 D flops per (query row, head, key it attends): q.k and p.v."""
        L = self.cache.context_lens.astype(np.int64)
        c = self.chunk_lens.astype(np.int64)
        keys = (c * L - c * (c - 1) // 2).sum()  # row i of a chunk attends L - c + i + 1 keys
        return int(4 * self.cache.head_size * self.cache.num_q_heads * keys)


def prefill(seed: int, cached_lens: Sequence[int], chunk_lens: Sequence[int], *,
            dtype: str = "bf16", num_q_heads: int = 8, num_kv_heads: int = 2,
            head_size: int = 128, block_size: int = 16, name: str = "prefill",
            **kw) -> PrefillWorkload:
    """Chunks of ``chunk_lens`` tokens after ``cached_lens`` cached tokens
    (0: a whole prompt).  Draw order: the cache workload's, then the query."""
    cached = np.asarray(cached_lens, dtype=np.int64)
    chunks = np.asarray(chunk_lens, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed))
    cache = _independent(name, rng, cached + chunks, dtype=dtype, num_q_heads=num_q_heads,
                         num_kv_heads=num_kv_heads, head_size=head_size,
                         block_size=block_size, **kw)
    starts = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    query = _normal(rng, (int(starts[-1]), num_q_heads, head_size), dtype)
    return PrefillWorkload(name=name, cache=cache, chunk_lens=chunks.astype(np.int32),
                           query_start=starts, query=query)


def prefill_opt13b(seed: int = 81011, num_seqs: int = 16, chunk: int = 512,
                   max_cached: int = 1536, block_size: int = 16) -> PrefillWorkload:
    """OPT-13B-shaped layer (40/40 heads, D 128, B 16, bf16): chunks of 512
    prompt tokens after 0 .. 1536 cached tokens (earlier chunks or prefix hits)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cached = rng.integers(0, max_cached + 1, size=num_seqs)
    return prefill(seed + 1, cached, np.full(num_seqs, chunk), num_q_heads=40, num_kv_heads=40,
                   head_size=128, block_size=block_size, name="prefill_opt13b")


def prefill_qwen2(seed: int = 81012, num_seqs: int = 32, max_chunk: int = 1024,
                  max_cached: int = 1024, block_size: int = 16) -> PrefillWorkload:
    """Qwen2-0.5B-shaped layer (14/2 heads, D 64, bf16): whole prompts and
    continuing chunks of 64 .. 1024 tokens after 0 .. 1024 cached tokens."""
    rng = np.random.Generator(np.random.PCG64(seed))
    chunks = rng.integers(64, max_chunk + 1, size=num_seqs)
    cached = np.where(rng.random(num_seqs) < 0.5, 0, rng.integers(0, max_cached + 1, size=num_seqs))
    return prefill(seed + 1, cached, chunks, num_q_heads=14, num_kv_heads=2, head_size=64,
                   block_size=block_size, name="prefill_qwen2")


PREFILL = {"prefill_opt13b": prefill_opt13b, "prefill_qwen2": prefill_qwen2}


NAMED = {
    "tiny": tiny,
    "opt13b_mha": opt13b_mha,
    "qwen2_gqa": qwen2_gqa,
    "shared_prefix": shared_prefix,
    "long_context": long_context,
}


def make(name: str, **kw) -> Workload:
    return NAMED[name](**kw)
