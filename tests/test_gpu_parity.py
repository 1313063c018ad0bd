"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer and copy work (slot mapping, write, gather) must be bit-exact; the
attention output must be within a per-row relative error of 2e-3 (bf16 inputs)
or 1e-5 (fp32 inputs): max over the row's dims of |gpu - oracle| divided by the
row's largest |oracle| value.
"""
from functools import lru_cache

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_81_amd as pkv
import workloads
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "opt13b_mha", "qwen2_gqa", "shared_prefix", "long_context"]


@lru_cache(maxsize=2)
def full(name):
    return workloads.make(name)


SMALL = {
    "tiny": lambda: workloads.tiny(),
    "opt13b_mha": lambda: workloads.opt13b_mha(num_seqs=4),
    "qwen2_gqa": lambda: workloads.qwen2_gqa(num_seqs=24),
    "shared_prefix": lambda: workloads.shared_prefix(num_prompts=2, forks=4, prompt_len=256,
                                                     max_private=40),
    "long_context": lambda: workloads.long_context(num_seqs=2, context_len=3000),
}


def oracle_pool(w):
    """The oracle's own pool: NaN, then every cached and new token written."""
    kv = H.nan_pool_numpy(w)
    slots = oracle.slot_mapping_ref(w.block_tables, w.cached_seq, w.cached_pos, w.block_size)
    oracle.write_ref(kv, w.cached_k, w.cached_v, slots)
    new = oracle.slot_mapping_ref(w.block_tables, np.arange(w.num_seqs), w.new_pos, w.block_size)
    oracle.write_ref(kv, w.new_k, w.new_v, new)
    return kv, slots, new


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- exact paths

@pytest.mark.parametrize("name", NAMES)
def test_slot_mapping_and_write_exact(name):
    w = full(name)
    say(f"[write] {name}: S={w.num_seqs} NB={w.num_blocks} cached={w.cached_k.shape[0]}")
    ref_kv, ref_cached, ref_new = oracle_pool(w)
    st = H.upload(w, fill=False, step=False)
    dev = st.kv.device
    got_cached = pkv.slot_mapping(st.tables, torch.from_numpy(w.cached_pos).to(dev), w.block_size,
                                  w.num_blocks, seq_ids=torch.from_numpy(w.cached_seq).to(dev))
    assert np.array_equal(got_cached.cpu().numpy(), ref_cached)
    H.fill_cached(st)
    H.run_write_step(st)
    assert np.array_equal(st.new_slots.cpu().numpy(), ref_new)
    got = H.to_numpy(st.kv)
    if w.dtype == "f32":
        got, ref_kv = got.view(np.uint32), ref_kv.view(np.uint32)
    assert np.array_equal(got, ref_kv), "pool differs from the oracle's write"


@pytest.mark.parametrize("name", NAMES)
def test_write_positions_exact(name):
    """Slot derivation and write in one launch: the same pool, bit for bit,
    and the same slots as the oracle's slot mapping and write."""
    w = full(name)
    say(f"[write positions] {name}: S={w.num_seqs} cached={w.cached_k.shape[0]}")
    ref_kv, ref_cached, ref_new = oracle_pool(w)
    st = H.upload(w, fill=False, step=False)
    dev = st.kv.device
    slots = torch.empty(w.cached_k.shape[0], dtype=torch.int64, device=dev)
    pkv.write_positions(H.to_torch(w.cached_k, w.dtype, dev), H.to_torch(w.cached_v, w.dtype, dev),
                        st.kv, st.tables, torch.from_numpy(w.cached_pos).to(dev),
                        seq_ids=torch.from_numpy(w.cached_seq).to(dev), slot_mapping=slots)
    assert np.array_equal(slots.cpu().numpy(), ref_cached)
    new = torch.empty(w.num_seqs, dtype=torch.int64, device=dev)
    pkv.write_positions(st.new_k, st.new_v, st.kv, st.tables, st.new_pos, slot_mapping=new)
    assert np.array_equal(new.cpu().numpy(), ref_new)
    got = H.to_numpy(st.kv)
    if w.dtype == "f32":
        got, ref_kv = got.view(np.uint32), ref_kv.view(np.uint32)
    assert np.array_equal(got, ref_kv), "pool differs from the oracle's write"


def test_write_positions_edge_cases():
    """Tokens whose slot is -1 (negative position, entry out of range,
    sequence absent, block past the table) write nothing."""
    dev = torch.device("cuda:0")
    tables = torch.tensor([[3, 5, -2**31], [7, -1, 99]], dtype=torch.int32, device=dev)
    seq = torch.tensor([0, 0, 0, 1, 1, 1, 2, -1, 0, 0], dtype=torch.int32, device=dev)
    pos = torch.tensor([0, 17, -1, 15, 16, 40, 0, 0, 48, 20], dtype=torch.int32, device=dev)
    kv = torch.full((2, 10, 16, 2, 64), float("nan"), dtype=torch.bfloat16, device=dev)
    k = torch.randn((10, 2, 64), device=dev).to(torch.bfloat16)
    v = torch.randn((10, 2, 64), device=dev).to(torch.bfloat16)
    slots = torch.empty(10, dtype=torch.int64, device=dev)
    pkv.write_positions(k, v, kv, tables, pos, seq_ids=seq, slot_mapping=slots)
    assert slots.cpu().tolist() == [48, 81, -1, 127, -1, -1, -1, -1, -1, 84]
    ref = torch.full_like(kv, float("nan"))
    flat = ref.view(2, 160, 2, 64)
    for t, sl in enumerate(slots.cpu().tolist()):
        if sl >= 0:
            flat[0, sl] = k[t]
            flat[1, sl] = v[t]
    assert torch.equal(kv.view(torch.int16), ref.view(torch.int16))


def test_slot_mapping_edge_cases():
    dev = torch.device("cuda:0")
    tables = torch.tensor([[3, 5, -2**31], [7, -1, 99]], dtype=torch.int32, device=dev)
    seq = torch.tensor([0, 0, 0, 1, 1, 1, 2, -1, 0], dtype=torch.int32, device=dev)
    pos = torch.tensor([0, 17, -1, 15, 16, 40, 0, 0, 48], dtype=torch.int32, device=dev)
    got = pkv.slot_mapping(tables, pos, 16, 10, seq_ids=seq).cpu().numpy()
    # -1: negative position, out-of-range entry (-1, 99), sequence 2 / -1 absent,
    # logical block past the table
    assert list(got) == [48, 81, -1, 127, -1, -1, -1, -1, -1]


@pytest.mark.parametrize("name", NAMES)
def test_gather_exact(name):
    w = SMALL[name]()
    ref_kv, _, _ = oracle_pool(w)
    st = H.upload(w)
    k, v = pkv.gather(st.kv, st.tables, st.lens, w.max_context_len)
    k, v = H.to_numpy(k), H.to_numpy(v)
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        rk, rv = oracle.gather_ref(ref_kv, w.block_tables[s], L)
        assert np.array_equal(k[s, :L].view(np.uint16), rk.view(np.uint16))
        assert np.array_equal(v[s, :L].view(np.uint16), rv.view(np.uint16))
        assert not k[s, L:].view(np.uint16).any() and not v[s, L:].view(np.uint16).any()
        # and the table view equals the generator's logical sequence
        lk, lv = w.logical_kv(s)
        assert np.array_equal(rk.view(np.uint16), lk.view(np.uint16))


# ---------------------------------------------------------------- attention

def _check_rows(got, ref, tol, what):
    err = H.row_rel_err(got, ref)
    worst = float(err.max()) if err.size else 0.0
    say(f"  {what}: worst row rel err {worst:.3e} (tol {tol:g})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert worst <= tol, f"{what}: worst row rel err {worst:.3e} > {tol}"


# fixed partition sizes checked besides the library's choice: the
# long-context shape's natural split into 512-token partitions
EXTRA_PARTITIONS = {"long_context": (512,)}


@pytest.mark.parametrize("name", NAMES)
def test_attention_small_full_oracle(name):
    w = SMALL[name]()
    ref_kv, _, _ = oracle_pool(w)
    ref = oracle.paged_attention_ref(w.query, ref_kv, w.block_tables, w.context_lens, w.scale, w.dtype)
    st = H.upload(w)
    unit = 32 if w.block_size <= 32 else w.block_size
    for P in sorted({w.partition_size, unit, 2 * unit, 0, *EXTRA_PARTITIONS.get(name, ())}):
        got = H.attend(st, partition_size=P).cpu().numpy()
        _check_rows(got, ref, H.tolerance(w), f"{name} P={P}")


@pytest.mark.parametrize("name", NAMES)
def test_attention_full_size_every_row(name):
    """Full-size workload in the benchmark's launch configuration (and at the
    extra fixed partition sizes): every output row of every sequence against
    the float64 oracle run over the oracle's own pool."""
    w = full(name)
    say(f"[attention] {name}: S={w.num_seqs} max_len={w.max_context_len}")
    st = H.upload(w)
    outs = {P: H.attend(st, partition_size=P).cpu().numpy()
            for P in (w.partition_size, *EXTRA_PARTITIONS.get(name, ()))}
    del st
    ref_kv, _, _ = oracle_pool(w)
    ref = oracle.paged_attention_ref(w.query, ref_kv, w.block_tables, w.context_lens, w.scale,
                                     w.dtype)
    del ref_kv
    for P, got in outs.items():
        _check_rows(got, ref, H.tolerance(w), f"{name} full size P={P}, all {w.num_seqs} sequences")


EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1024, 1025, 1500]


@pytest.mark.parametrize("D,B", [(128, 8), (128, 16), (128, 32), (128, 64), (64, 8), (64, 16),
                                 (64, 32), (64, 64)])
def test_attention_edge_lengths_bf16(D, B):
    w = workloads.custom(900 + D + B, EDGE_LENS, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                         head_size=D, block_size=B)
    ref_kv, _, _ = oracle_pool(w)
    ref = oracle.paged_attention_ref(w.query, ref_kv, w.block_tables, w.context_lens, w.scale, w.dtype)
    st = H.upload(w)
    for P in (0, 512, max(64, B)):
        got = H.attend(st, partition_size=P).cpu().numpy()
        assert not got[0].any(), "a sequence of length 0 must give zeros"
        _check_rows(got[1:], ref[1:], 2e-3, f"D={D} B={B} P={P}")


@pytest.mark.parametrize("P", [0, 64, 512])
def test_block_size_8_row_wise_keys(P):
    """Blocks of 8 tokens (a 16-token tile spans two blocks) with keys loaded
    row-wise through LDS (16 kv heads of 128 dims)."""
    w = workloads.custom(971, [1, 7, 8, 9, 33, 700, 1029], dtype="bf16", num_q_heads=16,
                         num_kv_heads=16, head_size=128, block_size=8)
    ref_kv, _, _ = oracle_pool(w)
    ref = oracle.paged_attention_ref(w.query, ref_kv, w.block_tables, w.context_lens, w.scale, w.dtype)
    got = H.attend(H.upload(w), partition_size=P).cpu().numpy()
    _check_rows(got, ref, 2e-3, f"B=8 row-wise keys P={P}")


@pytest.mark.parametrize("D,B", [(64, 16), (128, 8), (64, 48), (128, 1)])
def test_attention_fp32(D, B):
    w = workloads.custom(950 + D + B, [0, 1, 5, 47, 48, 49, 300, 777], dtype="f32",
                         num_q_heads=6, num_kv_heads=3, head_size=D, block_size=B)
    ref_kv, _, _ = oracle_pool(w)
    ref = oracle.paged_attention_ref(w.query, ref_kv, w.block_tables, w.context_lens, w.scale, w.dtype)
    st = H.upload(w)
    unit = int(np.lcm(32, B))
    for P in (0, unit, unit * (512 // unit)):
        got = H.attend(st, partition_size=P).cpu().numpy()
        assert not got[0].any()
        _check_rows(got[1:], ref[1:], 1e-5, f"fp32 D={D} B={B} P={P}")


def test_single_token_is_the_value_exactly():
    w = workloads.custom(31, [1, 1, 1], dtype="bf16", num_q_heads=16, num_kv_heads=4, head_size=128)
    st = H.upload(w)
    got = H.attend(st).cpu().numpy()
    v = H.to_numpy(st.new_v)  # the only token is the one written this step
    want = np.repeat(workloads.bf16_bits_to_f32(v), 4, axis=1)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("hq,hkv", [(1, 1), (16, 1), (48, 2), (20, 4), (40, 40)])
def test_attention_head_groupings(hq, hkv):
    w = workloads.custom(77 + hq, [5, 100, 700], dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                         head_size=128, block_size=16)
    ref_kv, _, _ = oracle_pool(w)
    ref = oracle.paged_attention_ref(w.query, ref_kv, w.block_tables, w.context_lens, w.scale, w.dtype)
    st = H.upload(w)
    _check_rows(H.attend(st, partition_size=256).cpu().numpy(), ref, 2e-3, f"Hq={hq} Hkv={hkv}")


def _oracle_rows(w, seqs):
    out = {}
    for s in seqs:
        k, v = w.logical_kv(s)
        out[s] = oracle.attention_ref(oracle.to_f64(w.query[s], w.dtype), oracle.to_f64(k, w.dtype),
                                      oracle.to_f64(v, w.dtype), w.scale)
    return out


@pytest.mark.parametrize("lens,hq,hkv,D", [
    ([100], 8, 1, 128),               # fewer stream steps than waves: one step per wave
    ([5000], 4, 4, 64),               # one sequence cut into hundreds of pieces
    ([3, 0, 40000, 17, 600], 32, 8, 128),  # a long context among short ones
])
def test_stream_schedule_cuts_and_merges(lens, hq, hkv, D):
    """The stream schedule (automatic partitioning) gives each wave an equal
    share of the batch's steps, so single contexts are cut into many pieces
    and merged; the rows agree with the oracle and repeat bit for bit."""
    w = workloads.custom(61 + len(lens), lens, dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                         head_size=D, block_size=16)
    st = H.upload(w)
    assert pkv.partition_size(w.num_seqs, hq, hkv, D, 16, w.max_context_len) == 0
    got = H.attend(st, partition_size=0).cpu().numpy()
    again = H.attend(st, partition_size=0).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))
    for s, ref in _oracle_rows(w, [s for s in range(w.num_seqs) if lens[s] > 0]).items():
        _check_rows(got[s], ref, 2e-3, f"stream seq {s} (L={lens[s]})")
    for s in range(w.num_seqs):
        if lens[s] == 0:
            assert not got[s].any()


def test_stream_schedule_full_batch_of_short_sequences():
    """511 sequences (the largest batch the stream schedule takes for one
    group of kv heads) of 1 to 80 tokens, GQA 14/2, head size 64."""
    rng = np.random.default_rng(21)
    lens = rng.integers(1, 81, 511)
    w = workloads.custom(22, lens, dtype="bf16", num_q_heads=14, num_kv_heads=2, head_size=64,
                         block_size=16)
    st = H.upload(w)
    assert pkv.partition_size(w.num_seqs, 14, 2, 64, 16, w.max_context_len) == 0
    got = H.attend(st, partition_size=0).cpu().numpy()
    ref_kv, _, _ = oracle_pool(w)
    ref = oracle.paged_attention_ref(w.query, ref_kv, w.block_tables, w.context_lens, w.scale, w.dtype)
    _check_rows(got, ref, 2e-3, "511 short sequences")


def test_stream_schedule_bad_sequences_and_bf16_output():
    w = workloads.custom(23, [40, 300, 700, 2], dtype="bf16", num_q_heads=8, num_kv_heads=2,
                         head_size=128, block_size=16)
    st = H.upload(w)
    clean = H.attend(st, partition_size=0).cpu().numpy()
    b16 = H.attend(st, partition_size=0, out_dtype=torch.bfloat16)
    f32 = H.attend(st, partition_size=0)
    assert torch.equal(f32.to(torch.bfloat16).view(torch.int16), b16.view(torch.int16))
    st.tables[1, 3] = w.num_blocks + 5     # outside the pool: the kernel must not read it
    bad = H.attend(st, partition_size=0).cpu().numpy()
    assert np.isnan(bad[1]).all()
    assert np.array_equal(bad[[0, 2, 3]].view(np.uint32), clean[[0, 2, 3]].view(np.uint32))
    st.lens[2] = w.table_width * 16 + 1     # longer than its table
    bad = H.attend(st, partition_size=0).cpu().numpy()
    assert np.isnan(bad[2]).all() and np.array_equal(bad[0], clean[0])


def test_stream_workspace_needs_no_clearing():
    """The stream schedule writes every workspace byte it later reads: a
    workspace full of garbage, or last used for another shape, gives the
    same bits as a zeroed one."""
    dev = torch.device("cuda:0")
    a = workloads.custom(71, [3000, 17, 900], dtype="bf16", num_q_heads=16, num_kv_heads=4,
                         head_size=128, block_size=16)
    b = workloads.custom(72, [5000, 2, 64, 1200, 333], dtype="bf16", num_q_heads=14,
                         num_kv_heads=2, head_size=64, block_size=32)
    sa, sb = H.upload(a), H.upload(b)
    need = max(pkv.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size,
                                   w.block_size, w.max_context_len) for w in (a, b))
    clean = torch.zeros(need, dtype=torch.uint8, device=dev)
    junk = torch.randint(0, 256, (need,), dtype=torch.uint8, device=dev)

    def run(st, ws):
        w = st.w
        return pkv.attention_decode(st.query, st.kv, st.tables, st.lens, w.scale, w.max_context_len,
                                    workspace=ws).cpu().numpy()

    ref_a, ref_b = run(sa, clean.clone()), run(sb, clean.clone())
    for st, ref in ((sa, ref_a), (sb, ref_b), (sa, ref_a), (sa, ref_a), (sb, ref_b)):
        got = run(st, junk)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    for s, r in _oracle_rows(b, [0, 3]).items():
        _check_rows(ref_b[s], r, 2e-3, f"stream seq {s}")


def test_many_partitions():
    w = workloads.custom(5, [16384, 9000], dtype="bf16", num_q_heads=8, num_kv_heads=1,
                         head_size=128, block_size=32)
    st = H.upload(w)
    got = H.attend(st, partition_size=32).cpu().numpy()
    for s in range(2):
        k, v = w.logical_kv(s)
        ref = oracle.attention_ref(oracle.to_f64(w.query[s], "bf16"), oracle.to_f64(k, "bf16"),
                                   oracle.to_f64(v, "bf16"), w.scale)
        _check_rows(got[s], ref, 2e-3, f"512 partitions, seq {s}")


# ---------------------------------------------------------------- invariants

def test_block_relabelling_is_bit_identical():
    w = workloads.qwen2_gqa(num_seqs=64)
    st = H.upload(w)
    base = H.attend(st).cpu().numpy()
    rng = np.random.default_rng(3)
    perm = rng.permutation(w.num_blocks)
    kv = H.to_numpy(st.kv)
    kv2 = np.empty_like(kv)
    kv2[:, perm] = kv
    t2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], w.block_tables).astype(np.int32)
    st.kv.copy_(H.to_torch(kv2, w.dtype, st.kv.device))
    st.tables.copy_(torch.from_numpy(t2).to(st.kv.device))
    again = H.attend(st).cpu().numpy()
    assert np.array_equal(base.view(np.uint32), again.view(np.uint32))


def test_shared_prefix_aliasing_is_bit_identical():
    w = workloads.shared_prefix(num_prompts=2, forks=8, prompt_len=512, max_private=64)
    st = H.upload(w)
    shared = H.attend(st).cpu().numpy()
    # give every fork a private copy of its prompt's blocks
    kv = H.to_numpy(st.kv)
    pb = 512 // 16
    extra = w.num_seqs * pb
    kv2 = np.concatenate([kv, np.zeros((2, extra) + kv.shape[2:], kv.dtype)], axis=1)
    t2 = w.block_tables.copy()
    for s in range(w.num_seqs):
        for j in range(pb):
            nb = w.num_blocks + s * pb + j
            kv2[:, nb] = kv[:, w.block_tables[s, j]]
            t2[s, j] = nb
    dev = st.kv.device
    private = pkv.attention_decode(st.query, H.to_torch(kv2, w.dtype, dev), torch.from_numpy(t2).to(dev),
                                   st.lens, w.scale, w.max_context_len).cpu().numpy()
    assert np.array_equal(shared.view(np.uint32), private.view(np.uint32))


@pytest.mark.parametrize("name", ["shared_prefix", "qwen2_gqa"])
def test_cached_and_streamed_loads_agree_bit_for_bit(name):
    w = SMALL[name]()
    st = H.upload(w)
    a = H.attend(st, shared_blocks=False).cpu().numpy()
    b = H.attend(st, shared_blocks=True).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_result_does_not_depend_on_work_split():
    """The same partition size with a different number of partitions per
    workgroup gives identical rows: 16 sequences of 16384 tokens make the
    launcher give each wave two 512-token partitions, one sequence alone one."""
    w = workloads.long_context(num_seqs=16, context_len=16384, partition_size=512)
    st = H.upload(w)
    two = H.attend(st).cpu().numpy()
    one = pkv.attention_decode(st.query[:1].contiguous(), st.kv, st.tables[:1].contiguous(),
                               st.lens[:1].contiguous(), w.scale, w.max_context_len,
                               partition_size=512).cpu().numpy()
    assert np.array_equal(one[0].view(np.uint32), two[0].view(np.uint32))


def test_compact_item_list_matches_dense_grid_bit_for_bit():
    """A batch of at most 512 sequences whose contexts span several workgroup
    runs walks a compact list of work items; a larger one uses the dense grid.
    The first 64 sequences of a 600-sequence batch give the same bits either
    way -- also with 32-token partitions, where each workgroup of the compact
    launch takes many items -- and agree with the oracle."""
    rng = np.random.default_rng(12)
    lens = rng.integers(16, 1200, 600)
    w = workloads.custom(13, lens, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_size=128,
                         block_size=16)
    st = H.upload(w)
    n = 64
    sub = [t[:n].contiguous() for t in (st.query, st.tables, st.lens)]
    for P in (32, 256):
        say(f"[compact] P={P}")
        dense = H.attend(st, partition_size=P).cpu().numpy()[:n]
        compact = pkv.attention_decode(*sub[:1], st.kv, *sub[1:], w.scale, int(lens[:n].max()),
                                       partition_size=P).cpu().numpy()
        assert np.array_equal(dense.view(np.uint32), compact.view(np.uint32)), f"P={P}"
    for s in (0, int(np.argmax(lens[:n])), int(np.argmin(lens[:n])), 40):
        k, v = w.logical_kv(s)
        ref = oracle.attention_ref(oracle.to_f64(w.query[s], "bf16"), oracle.to_f64(k, "bf16"),
                                   oracle.to_f64(v, "bf16"), w.scale)
        _check_rows(compact[s], ref, 2e-3, f"compact seq {s} (L={lens[s]})")


def test_bf16_output_is_rounded_fp32_output():
    w = workloads.long_context(num_seqs=2, context_len=2000)
    st = H.upload(w)
    f32 = H.attend(st)
    b16 = H.attend(st, out_dtype=torch.bfloat16)
    assert torch.equal(f32.to(torch.bfloat16).view(torch.int16), b16.view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bad_table_entry_poisons_only_its_sequence(dtype):
    w = workloads.custom(8, [40, 300, 700], dtype=dtype, num_q_heads=4, num_kv_heads=2,
                         head_size=64, block_size=16)
    st = H.upload(w)
    clean = H.attend(st, partition_size=64).cpu().numpy()
    st.tables[1, 3] = w.num_blocks + 5     # outside the pool: the kernel must not read it
    bad = H.attend(st, partition_size=64).cpu().numpy()
    assert np.isnan(bad[1]).all()
    assert np.array_equal(bad[[0, 2]], clean[[0, 2]])
    st.lens[2] = w.table_width * 16 + 1     # longer than its table
    bad = H.attend(st, partition_size=64).cpu().numpy()
    assert np.isnan(bad[2]).all() and np.array_equal(bad[0], clean[0])


def test_write_skips_invalid_slots():
    w = workloads.custom(9, [3, 20], dtype="bf16", num_q_heads=2, num_kv_heads=2, head_size=64)
    st = H.upload(w)
    before = H.to_numpy(st.kv).copy()
    slots = torch.tensor([-1, w.num_blocks * w.block_size], dtype=torch.int64, device=st.kv.device)
    pkv.write(st.new_k, st.new_v, st.kv, slots)
    assert np.array_equal(H.to_numpy(st.kv), before)
