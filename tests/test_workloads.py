"""The seeded input generators: reproducible, well-formed, shaped as stated."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e38, 1e-40], np.float32)])
    ours = workloads.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(workloads.bf16_bits_to_f32(ours),
                          torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def _check_structure(w, shared_ok=False):
    S, B, NB = w.num_seqs, w.block_size, w.num_blocks
    assert w.block_tables.dtype == np.int32 and w.context_lens.dtype == np.int32
    owner = {}
    for s in range(S):
        L = int(w.context_lens[s])
        nb = oracle.blocks_needed(L, B)
        row = w.block_tables[s]
        assert np.all((row[:nb] >= 0) & (row[:nb] < NB))
        assert np.all(row[nb:] == workloads.TABLE_PAD)
        assert w.logical_rows(s).shape[0] == L
        for j, b in enumerate(row[:nb]):
            owner.setdefault(int(b), set()).add((s, j))
        assert w.new_pos[s] in (L - 1, -1)
    if not shared_ok:
        assert all(len(v) == 1 for v in owner.values())
    # every row written before or during the step has its own slot
    writers = np.nonzero(w.new_pos >= 0)[0]
    slots = np.concatenate([
        oracle.slot_mapping_ref(w.block_tables, w.cached_seq, w.cached_pos, B),
        oracle.slot_mapping_ref(w.block_tables, writers, w.new_pos[writers], B)])
    assert slots.min() >= 0 and slots.max() < NB * B
    assert np.unique(slots).shape[0] == slots.shape[0]
    # each sequence's positions 0..L-1 are covered exactly once by its rows
    n = w.cached_k.shape[0]
    for s in range(S):
        rows = w.logical_rows(s)
        pos = np.where(rows < n, w.cached_pos[np.minimum(rows, max(n - 1, 0))], w.new_pos[s])
        assert np.array_equal(pos, np.arange(w.context_lens[s]))


def test_tiny():
    w = workloads.tiny()
    assert list(w.context_lens) == [7, 33, 100, 250]
    assert w.num_blocks == 64 and w.dtype == "f32" and w.scale == 0.125
    assert sum(oracle.blocks_needed(int(n), 16) for n in w.context_lens) == 27
    _check_structure(w)


def test_reproducible():
    a = workloads.custom(123, [5, 40, 0, 1], dtype="bf16", num_q_heads=4, num_kv_heads=2)
    b = workloads.custom(123, [5, 40, 0, 1], dtype="bf16", num_q_heads=4, num_kv_heads=2)
    for f in ("block_tables", "query", "cached_k", "cached_v", "new_k", "new_v", "seq_rows"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    _check_structure(a)
    assert a.new_pos[2] == -1 and a.logical_rows(2).shape[0] == 0


def test_qwen2_gqa_full_size():
    w = workloads.qwen2_gqa()
    L = w.context_lens
    assert w.num_seqs == 256 and L.min() >= 16 and L.max() <= 8192
    assert 300 < np.median(L) < 900  # median 512 in distribution
    assert (w.num_q_heads, w.num_kv_heads, w.head_size, w.block_size) == (14, 2, 64, 16)
    needed = sum(oracle.blocks_needed(int(n), 16) for n in L)
    assert w.num_blocks == int(np.ceil(1.25 * needed))
    _check_structure(w)


def test_shared_prefix_full_size():
    w = workloads.shared_prefix()
    assert w.num_seqs == 256
    L = w.context_lens
    assert L.min() >= 1024 and L.max() <= 1280
    for p in range(32):
        rows = w.block_tables[p * 8:(p + 1) * 8, :64]
        assert np.all(rows == rows[0])          # the prompt's blocks are aliased
    _check_structure(w, shared_ok=True)
    # the prompt's K/V are one copy shared by all forks
    k0, _ = w.logical_kv(0)
    k7, _ = w.logical_kv(7)
    assert np.array_equal(k0[:1024], k7[:1024])
    assert np.all((w.new_pos == -1) == (L == 1024))


@pytest.mark.parametrize("kw", [dict(num_seqs=6), dict(num_seqs=3, lo=16, hi=300)])
def test_opt13b_reduced(kw):
    w = workloads.opt13b_mha(**kw)
    assert w.context_lens.min() >= kw.get("lo", 256) and w.context_lens.max() <= kw.get("hi", 2048)
    assert (w.num_q_heads, w.num_kv_heads, w.head_size, w.block_size) == (40, 40, 128, 16)
    _check_structure(w)


def test_long_context_reduced():
    w = workloads.long_context(num_seqs=2, context_len=2048)
    assert w.num_blocks == 2 * 64 and w.block_size == 32 and w.partition_size == 0
    _check_structure(w)
