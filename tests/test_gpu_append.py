"""A decode step with its write in one call (paged_attention_decode_append).

Its contract is the pair it replaces: the cache and the output must be
bit-identical to paged_kv_write_positions (each sequence's new token at
position context_lens[s] - 1) followed by paged_attention_decode -- under
the stream schedule, where the attention launch stores the new rows itself,
and on the other schedules, where the library launches the write first.  The
output is also checked against the oracle on the oracle's own pool.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_81_amd as pkv
import workloads
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def _separate(st, P, max_len, shared=False, out_dtype=torch.float32):
    pos = (st.lens - 1).to(torch.int32)
    pkv.write_positions(st.new_k, st.new_v, st.kv, st.tables, pos)
    return pkv.attention_decode(st.query, st.kv, st.tables, st.lens, st.w.scale, max_len,
                                partition_size=P, shared_blocks=shared, out_dtype=out_dtype)


def _fused(st, P, max_len, shared=False, out_dtype=torch.float32):
    return pkv.attention_decode_append(st.query, st.new_k, st.new_v, st.kv, st.tables, st.lens,
                                       st.w.scale, max_len, partition_size=P, shared_blocks=shared,
                                       out_dtype=out_dtype)


def _compare(w, P=0, max_len=None, shared=False, out_dtype=torch.float32, oracle_check=True):
    """Fused and separate calls on two copies of the same pool; returns the output."""
    max_len = w.max_context_len if max_len is None else max_len
    a = H.upload(w, step=False)
    b = H.upload(w, step=False)
    got = _fused(a, P, max_len, shared, out_dtype)
    ref = _separate(b, P, max_len, shared, out_dtype)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(a.kv), _bits(b.kv)), "caches differ"
    assert np.array_equal(_bits(got), _bits(ref)), "outputs differ"
    if oracle_check:
        kv = H.nan_pool_numpy(w)
        slots = oracle.slot_mapping_ref(w.block_tables, w.cached_seq, w.cached_pos, w.block_size)
        oracle.write_ref(kv, w.cached_k, w.cached_v, slots)
        new = oracle.slot_mapping_ref(w.block_tables, np.arange(w.num_seqs), w.new_pos,
                                      w.block_size)
        oracle.write_ref(kv, w.new_k, w.new_v, new)
        exp = oracle.paged_attention_ref(w.query, kv, w.block_tables, w.context_lens, w.scale,
                                         w.dtype)
        err = H.row_rel_err(got.float().cpu().numpy(), exp)
        say(f"  worst row rel err {float(err.max()):.3e}")
        assert float(err.max()) <= H.tolerance(w)
    return got


EDGE = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1000]


@pytest.mark.parametrize("hq,hkv,D,B", [(8, 8, 128, 16), (14, 2, 64, 16), (32, 8, 128, 32),
                                         (40, 2, 128, 16), (8, 2, 64, 8), (4, 4, 128, 64)])
def test_stream_append_matches_write_then_decode(hq, hkv, D, B):
    """Stream schedule (library's choice on these small batches): edge lengths,
    MHA and GQA, more than 16 query heads per kv head (two column chunks)."""
    w = workloads.custom(9100 + hq + D + B, EDGE, num_q_heads=hq, num_kv_heads=hkv,
                         head_size=D, block_size=B)
    assert pkv.partition_size(w.num_seqs, hq, hkv, D, B, w.max_context_len, 0, torch.bfloat16) == 0
    say(f"[append] stream hq={hq} hkv={hkv} D={D} B={B}")
    _compare(w)


@pytest.mark.parametrize("P", [32, 64, 512])
def test_fixed_partitions_append_matches_write_then_decode(P):
    """Fixed partitions: the library launches the write, then the attention."""
    w = workloads.custom(9200 + P, EDGE, num_q_heads=16, num_kv_heads=4, head_size=128,
                         block_size=16)
    say(f"[append] fixed P={P}")
    _compare(w, P=P)


def test_fp32_append_matches_write_then_decode():
    w = workloads.tiny()
    say("[append] fp32 tiny")
    _compare(w)


# fp32 caches store the new token inside the attention launch: head shapes,
# blocks of 5 and 48 tokens, partitions whose last token lies past their
# first 64 (its block then comes from a table load of its own), two chunks of
# query heads per kv head (both store the row)
@pytest.mark.parametrize("hq,hkv,D,B,P", [(4, 4, 64, 16, 64), (40, 2, 128, 5, 320),
                                          (6, 3, 64, 48, 96), (8, 2, 128, 16, 512),
                                          (12, 4, 64, 8, 0)])
def test_fp32_append_shapes(hq, hkv, D, B, P):
    w = workloads.custom(9600 + hq + D + B, [1, 2, 17, 64, 65, 130, 300, 511, 700],
                         dtype="f32", num_q_heads=hq, num_kv_heads=hkv, head_size=D,
                         block_size=B)
    say(f"[append] fp32 {hq}/{hkv} D={D} B={B} P={P}")
    assert pkv.lib.paged_attention_append_in_launch(w.num_seqs, hq, hkv, D, B,
                                                     w.max_context_len, P, 0) == 1
    _compare(w, P=P)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_edge_cases(dtype):
    """A length-0 sequence (nothing written, zeros), an out-of-range table
    entry for a new token's block (NaN, nothing written), a sequence longer
    than max_context_len (its token is still written, as the write kernel
    does; NaN under the bf16 stream schedule, which checks that bound, and
    attended normally by the fp32 kernel, whose fixed partitions still cover
    it) and bf16 output: all exactly as the separate calls."""
    w = workloads.custom(9300, [0, 40, 33, 100, 17, 64], dtype=dtype, num_q_heads=8,
                         num_kv_heads=2, head_size=64, block_size=16)
    w.block_tables[1, (40 - 1) // 16] = w.num_blocks + 7   # new token's block out of range
    w.block_tables[4, (17 - 1) // 16] = -3                 # ... and negative
    say("[append] edge cases")
    got = _compare(w, max_len=80, oracle_check=False)
    out = got.cpu().numpy()
    assert np.all(out[0] == 0)
    for s in (1, 3, 4) if dtype == "bf16" else (1, 4):
        assert np.all(np.isnan(out[s])), s
    assert np.all(np.isfinite(out[[2, 5] if dtype == "bf16" else [2, 3, 5]]))
    _compare(w, max_len=80, out_dtype=torch.bfloat16, oracle_check=False)


@pytest.mark.parametrize("name", ["opt13b_mha", "qwen2_gqa", "long_context"])
def test_full_size_append_matches_write_then_decode(name):
    """The benchmark's workloads at full size, in its launch configuration."""
    w = workloads.make(name)
    say(f"[append] full size {name}")
    _compare(w, P=w.partition_size, oracle_check=False)


def test_append_partitions_then_merge_and_repeat():
    """The two-launch form gives the one-call result, and calling again (the
    row already stored) changes nothing."""
    w = workloads.qwen2_gqa(num_seqs=40)
    st = H.upload(w, step=False)
    one = pkv.attention_decode_append(st.query, st.new_k, st.new_v, st.kv, st.tables, st.lens,
                                      w.scale, w.max_context_len)
    ws = torch.empty(pkv.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size,
                                         w.block_size, w.max_context_len, 0, st.kv.dtype),
                     dtype=torch.uint8, device=st.kv.device)
    out = torch.empty_like(one)
    pkv.attention_append_partitions(st.query, st.new_k, st.new_v, st.kv, st.tables, st.lens,
                                    w.scale, w.max_context_len, out=out, workspace=ws)
    pkv.attention_merge(st.query, st.kv, st.tables, st.lens, w.scale, w.max_context_len,
                        out=out, workspace=ws)
    assert np.array_equal(_bits(one), _bits(out))


def test_write_placement_for_the_benchmark_shapes():
    """Where the write goes on this device: inside the attention launch for
    the Qwen2-shaped and long-context batches (few pieces hold a sequence's
    last step) and for fp32 caches, a launch of its own for the OPT-13B-shaped
    one."""
    want = {"qwen2_gqa": 1, "long_context": 1, "opt13b_mha": 0, "tiny": 1}
    for name, exp in want.items():
        w = workloads.make(name)
        got = pkv.lib.paged_attention_append_in_launch(
            w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size, w.block_size,
            w.max_context_len, w.partition_size, 1 if w.dtype == "bf16" else 0)
        assert got == exp, (name, got)


def test_two_launch_form_when_the_write_goes_first():
    """On a batch where the library launches the write before the attention
    (many units per piece), the two-launch form still equals the one call and
    the separate calls."""
    w = workloads.opt13b_mha(num_seqs=64)
    assert pkv.lib.paged_attention_append_in_launch(
        w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size, w.block_size,
        w.max_context_len, 0, 1) == 0
    a = H.upload(w, step=False)
    b = H.upload(w, step=False)
    one = pkv.attention_decode_append(a.query, a.new_k, a.new_v, a.kv, a.tables, a.lens,
                                      w.scale, w.max_context_len)
    ws = torch.empty(pkv.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size,
                                         w.block_size, w.max_context_len, 0, b.kv.dtype),
                     dtype=torch.uint8, device=b.kv.device)
    two = torch.empty_like(one)
    pkv.attention_append_partitions(b.query, b.new_k, b.new_v, b.kv, b.tables, b.lens, w.scale,
                                    w.max_context_len, out=two, workspace=ws)
    pkv.attention_merge(b.query, b.kv, b.tables, b.lens, w.scale, w.max_context_len, out=two,
                        workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(a.kv), _bits(b.kv))
    assert np.array_equal(_bits(one), _bits(two))


@pytest.mark.parametrize("seed", range(8))
def test_append_random_batches(seed):
    """Seeded random batches (batch size, length mix, head grouping, head and
    block size): cache and output bit-identical to the separate calls, and a
    sample of sequences against the oracle."""
    rng = np.random.default_rng(9400 + seed)
    hq, hkv = [(8, 8), (14, 2), (32, 8), (40, 2), (12, 4), (16, 1)][seed % 6]
    D = [64, 128][seed % 2]
    B = [8, 16, 32][seed % 3]
    S = int(rng.integers(1, 300))
    lens = np.maximum(1, np.round(rng.lognormal(np.log(300), 1.2, size=S))).astype(int)
    lens = np.minimum(lens, 4000)
    lens[rng.random(S) < 0.1] = 1
    w = workloads.custom(9500 + seed, lens.tolist(), num_q_heads=hq, num_kv_heads=hkv,
                         head_size=D, block_size=B)
    say(f"[append] random seed={seed} S={S} hq={hq} hkv={hkv} D={D} B={B} "
        f"in_launch={pkv.lib.paged_attention_append_in_launch(S, hq, hkv, D, B, w.max_context_len, 0, 1)}")
    got = _compare(w, oracle_check=False).cpu().numpy()
    for s in sorted({int(np.argmax(w.context_lens)), int(rng.integers(0, S))}):
        k, v = w.logical_kv(s)
        ref = oracle.attention_ref(oracle.to_f64(w.query[s], w.dtype), oracle.to_f64(k, w.dtype),
                                   oracle.to_f64(v, w.dtype), w.scale)
        err = float(H.row_rel_err(got[s], ref).max())
        assert err <= H.tolerance(w), (s, err)
