"""Plain, slow, float64 reference for one paged decode step.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed, and from where:

* The cache of one layer is a single array ``kv[2, NB, B, Hkv, D]``; index 0 of
  the first axis holds keys, index 1 values; the block id is the index on the
  second axis [walkthrough, "BlockPoolの生成過程" (how the block pool and the
  per-layer tensors are built): the reshaped tensor and what its axes mean].
* A sequence's tokens fill its logical blocks left to right; token ``t`` lives
  in logical block ``t // B`` at offset ``t % B`` [explainer, section 2 (block
  table and logical-to-physical translation), the ``BlockTable`` sketch]; the
  block table maps each logical block to a physical one [review, "vLLM의 메모리
  관리" (memory management)].
* Attention over a sequence reads its keys/values block by block through the
  table, scores the query against the keys, weights the values and combines
  the per-block pieces into the output [review, "PagedAttention" section;
  notes, "KV Cache 管理器" (the algorithm figure's description)].  Paging
  changes only *where* K/V live, so the result is ordinary softmax attention
  over the sequence's tokens in logical order; that is what this module
  computes, in float64.

Readings where the pages are silent (each also listed in the design notes):

1. slot = physical_block * B + offset (the pages give ``//`` and ``%`` and the
   [num_blocks, block_size] axes, not the flattening);
2. a negative slot means "write nothing";
3. ``L_s`` counts the token appended this step, at position ``L_s - 1``;
4. scores are scaled by ``scale`` (1/sqrt(D) in every workload);
5. query head ``h`` reads kv head ``h // G`` with ``G = Hq / Hkv``
   (contiguous groups);
6. a sequence with ``L_s == 0`` attends to nothing and its output is zero;
7. a split into partitions of ``P`` tokens is merged by the log-sum-exp rule
   (the pages do not describe a split; it is an exact identity);
8. a chunk of query tokens (prefill) is the last tokens of its sequence, its
   own K/V already in the cache, and each of its tokens attends causally.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

TABLE_PAD = -2**31  # table entries past a sequence's last block hold this


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen inputs to float64: bf16 bit patterns (uint16) or float32 values.

    A bf16 pattern is the upper half of the float32 with the same value, so the
    widening is exact.
    """
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------- block arithmetic

def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Physical blocks a request of ``num_tokens`` tokens holds.

    [walkthrough, "ブロック割当のロジック" (block allocation logic)]: the count is
    the ceiling of tokens over block size (10 tokens at size 16 take one
    block; 50 take four).  [review, "물리적 블록 할당" (physical block
    allocation)]: blocks fill left to right and a new block is taken only when
    the last one is full, so this is also the count a growing sequence holds.
    """
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("bad sizes")
    whole, rest = divmod(num_tokens, block_size)
    return whole + (1 if rest else 0)


def last_block_fill(num_tokens: int, block_size: int) -> int:
    """Tokens held by a sequence's last block (the table's "#filled" record).

    [review, the first and second decoding steps of the worked example]: the
    table records how many slots of each block are filled; only the last block
    can be partly filled.
    """
    if num_tokens == 0:
        return 0
    return num_tokens - (blocks_needed(num_tokens, block_size) - 1) * block_size


def slot_of(table_row: Sequence[int], position: int, block_size: int) -> int:
    """Physical slot of token ``position`` of a sequence.

    [explainer, section 2, ``BlockTable.append_token``]: the logical block is
    ``position // B`` and the offset inside it ``position % B``; the table row
    names the physical block.  Reading 1: the slot is
    ``physical * B + offset``.  Reading 2: a negative position has no slot (-1).
    """
    if position < 0:
        return -1
    logical_block, offset = divmod(int(position), block_size)
    physical = int(table_row[logical_block])
    return physical * block_size + offset


def slot_mapping_ref(block_tables: np.ndarray, seq_ids: np.ndarray, positions: np.ndarray,
                     block_size: int) -> np.ndarray:
    """``slot_mapping`` for a list of (sequence, position) pairs.

    [walkthrough, "ブロックアロケーションの基本概念" (basic concepts of block
    allocation), last paragraph]: in the decode phase a ``slot_mapping`` tensor
    records, for each newly generated token, which slot of the physical cache
    it occupies.
    """
    seq_ids = np.asarray(seq_ids)
    positions = np.asarray(positions)
    out = np.full(positions.shape[0], -1, dtype=np.int64)
    ok = positions >= 0
    logical_block, offset = np.divmod(positions[ok].astype(np.int64), block_size)
    physical = block_tables[seq_ids[ok].astype(np.int64), logical_block].astype(np.int64)
    out[ok] = physical * block_size + offset
    return out


# ---------------------------------------------------------------- write and gather

def write_ref(kv: np.ndarray, k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray) -> None:
    """Store each token's K and V at its slot (in place; an exact copy).

    [review, "디코딩 과정" (decoding)]: newly generated KV is stored into
    physical KV blocks; [walkthrough, basic concepts]: ``slot_mapping`` names
    the slot.  ``kv`` is ``[2, NB, B, Hkv, D]``; ``k`` and ``v`` are
    ``[T, Hkv, D]`` in the same element representation.  Reading 2: a negative
    slot writes nothing.  Slots must be distinct.
    """
    B = kv.shape[2]
    slot_mapping = np.asarray(slot_mapping, dtype=np.int64)
    sel = slot_mapping >= 0
    block, offset = np.divmod(slot_mapping[sel], B)
    kv[0, block, offset] = k[sel]
    kv[1, block, offset] = v[sel]


def gather_ref(kv: np.ndarray, table_row: np.ndarray, context_len: int) -> Tuple[np.ndarray, np.ndarray]:
    """Read one sequence's K and V, in logical order, through its block table.

    [walkthrough, "ブロック割当のロジック"]: each layer's cache is accessed as
    ``kv[:, table, ...]``; [explainer, section 2]: token ``t`` is at offset
    ``t % B`` of logical block ``t // B``.  Entries past the last block are
    never read.  Returns ``[L, Hkv, D]`` arrays in ``kv``'s representation.
    """
    B = kv.shape[2]
    pos = np.arange(context_len, dtype=np.int64)
    logical_block, offset = np.divmod(pos, B)
    physical = np.asarray(table_row, dtype=np.int64)[logical_block]
    return kv[0, physical, offset], kv[1, physical, offset]


# ---------------------------------------------------------------- attention

def _scores(q_h: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    return scale * (keys @ q_h)


def attention_ref(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one decoding token over its sequence (float64).

    [review, "PagedAttention" section; notes, the algorithm figure]: the query
    is multiplied with every key to give the scores, the scores weight the
    values, and the weighted values are summed into the output.  Softmax
    normalises the weights (textbook attention).  ``q`` is ``[Hq, D]``,
    ``keys``/``values`` are ``[L, Hkv, D]`` float64.  Readings 4-6: scale,
    head grouping ``h // G``, zero output for ``L == 0``.
    """
    Hq, D = q.shape
    L, Hkv, _ = keys.shape
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    group = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    if L == 0:
        return out
    for h in range(Hq):
        g = h // group
        z = _scores(q[h], keys[:, g, :], scale)
        w = np.exp(z - z.max())
        out[h] = (w / w.sum()) @ values[:, g, :]
    return out


def paged_attention_ref(query: np.ndarray, kv: np.ndarray, block_tables: np.ndarray,
                        context_lens: np.ndarray, scale: float, dtype: str,
                        seqs: Sequence[int] = None) -> np.ndarray:
    """Decode attention for a batch: gather each sequence through its table,
    then attend (float64).  Returns ``[S, Hq, D]`` (rows not in ``seqs`` zero).
    """
    S, Hq, D = query.shape
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        k, v = gather_ref(kv, block_tables[s], int(context_lens[s]))
        out[s] = attention_ref(to_f64(query[s], dtype), to_f64(k, dtype), to_f64(v, dtype), scale)
    return out


# ---------------------------------------------------------------- prefill / chunked prefill

def chunk_positions(context_len: int, chunk_len: int) -> np.ndarray:
    """Positions of a chunk of ``chunk_len`` query tokens that ends a sequence
    of ``context_len`` tokens: ``context_len - chunk_len .. context_len - 1``.

    Reading 8: a chunk's own K/V is in the cache when it attends (as the decode
    token's is, reading 3), so the chunk is the last ``chunk_len`` tokens of
    the sequence.  Positions restart at 0 for every sequence of a batch
    [walkthrough, "ブロックアロケーションの基本概念" (basics of block
    allocation): concatenated prompts keep their own position ids].
    """
    if chunk_len > context_len or chunk_len < 0:
        raise ValueError("a chunk cannot be longer than its sequence")
    return np.arange(context_len - chunk_len, context_len, dtype=np.int64)


def prefill_attention_ref(query: np.ndarray, kv: np.ndarray, block_tables: np.ndarray,
                          context_lens: np.ndarray, query_start: np.ndarray, scale: float,
                          dtype: str) -> np.ndarray:
    """Causal attention of chunks of query tokens over their paged sequences
    (float64): the prompt (prefill) step, and chunked prefill.

    [review, "프리필(Prefill) 단계" (prefill stage)]: a prompt is processed with
    ordinary self-attention, each token attending to itself and the tokens
    before it; [review, "디코딩 과정" (the decoding process)]: the input
    tokens of all requests of an iteration are joined into one sequence and
    the kernel reads earlier K/V through the block tables;
    [walkthrough, "ブロックアロケーションの基本概念"]: an attention mask keeps
    each joined sequence to itself.

    ``query`` is ``[T, Hq, D]``: rows ``query_start[s] .. query_start[s+1]-1``
    are sequence ``s``'s chunk, whose tokens sit at :func:`chunk_positions`.
    The token at position ``p`` attends to the sequence's keys ``0 .. p``.
    Returns ``[T, Hq, D]``.
    """
    T = query.shape[0]
    out = np.zeros(query.shape, dtype=np.float64)
    for s in range(len(context_lens)):
        r0, r1 = int(query_start[s]), int(query_start[s + 1])
        L = int(context_lens[s])
        pos = chunk_positions(L, r1 - r0)
        k, v = gather_ref(kv, block_tables[s], L)
        k, v = to_f64(k, dtype), to_f64(v, dtype)
        for i, p in enumerate(pos):
            out[r0 + i] = attention_ref(to_f64(query[r0 + i], dtype), k[:p + 1], v[:p + 1], scale)
    assert r1 <= T
    return out


# ---------------------------------------------------------------- context partitions

def partition_stats_ref(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
                        partition: int) -> List[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """Per-partition softmax statistics for the split of the context.

    Partition ``p`` covers positions ``[p*P, min((p+1)*P, L))``.  For each it
    returns ``(m, l, o)`` per query head: the largest score, the sum of
    ``exp(score - m)``, and the attention output over that partition alone.
    Reading 7 (the pages do not describe a split).
    """
    L = keys.shape[0]
    Hq = q.shape[0]
    group = Hq // keys.shape[1]
    stats = []
    for start in range(0, L, partition):
        stop = min(L, start + partition)
        m = np.empty(Hq)
        l = np.empty(Hq)
        o = np.empty((Hq, q.shape[1]))
        for h in range(Hq):
            g = h // group
            z = _scores(q[h], keys[start:stop, g, :], scale)
            m[h] = z.max()
            w = np.exp(z - m[h])
            l[h] = w.sum()
            o[h] = (w / l[h]) @ values[start:stop, g, :]
        stats.append((m, l, o))
    return stats


def merge_ref(stats: List[Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> np.ndarray:
    """Merge partition statistics into the full-context output.

    With ``M = max_p m_p`` and ``w_p = l_p * exp(m_p - M)`` the output is
    ``sum_p w_p o_p / sum_p w_p`` (log-sum-exp merge; exact in real
    arithmetic).  Reading 7.
    """
    ms = np.stack([m for m, _, _ in stats])
    ls = np.stack([l for _, l, _ in stats])
    os_ = np.stack([o for _, _, o in stats])
    big_m = ms.max(axis=0)
    w = ls * np.exp(ms - big_m)
    return (w[:, :, None] * os_).sum(axis=0) / w.sum(axis=0)[:, None]


# ---------------------------------------------------------------- pool sizing

def page_bytes(block_size: int, num_kv_heads: int, head_size: int, dtype_bytes: int) -> int:
    """Bytes of one block of one layer: (K+V) x block x kv heads x head size x dtype.

    [walkthrough, "ブロックアロケーションの基本概念"].
    """
    return 2 * block_size * num_kv_heads * head_size * dtype_bytes


def num_blocks_for(available_bytes: int, page: int, num_layers: int) -> int:
    """Blocks that fit: available memory divided by page size times layers.

    [walkthrough, "ブロックアロケーションの基本概念"]: the block count is the
    usable memory divided by the page size and the number of layers.
    """
    return available_bytes // (page * num_layers)


def cache_shape_from_bytes(tensor_bytes: int, block_size: int, num_kv_heads: int,
                           head_size: int, dtype_bytes: int) -> Tuple[int, int, int, int, int]:
    """Shape a raw per-layer byte tensor takes after the reshape.

    [walkthrough, "BlockPoolの生成過程"]: each layer's raw int8 tensor is
    reshaped to ``[2, num_blocks, block_size, num_kv_heads, head_size]``.
    """
    per_block = page_bytes(block_size, num_kv_heads, head_size, dtype_bytes)
    if tensor_bytes % per_block:
        raise ValueError("tensor is not a whole number of pages")
    return (2, tensor_bytes // per_block, block_size, num_kv_heads, head_size)


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_size: int, dtype_bytes: int) -> int:
    """KV bytes one token occupies across all layers (K and V).

    [review, "vLLM의 기존 문제점" (the problem): the OPT-13B example].
    """
    return 2 * num_layers * num_kv_heads * head_size * dtype_bytes

