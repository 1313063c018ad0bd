"""The C ABI library loads and exports what include/paged_kv.h declares; the
host-side argument checks and sizing helpers behave.  Nothing here launches a
kernel, so it runs without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_kv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("paged_kv_write", "paged_attention_decode", "paged_kv_slot_mapping",
                     "paged_kv_gather", "pkv_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    from paged_kv_cache_81_amd import _lib
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared but not exported"
    assert sorted(_lib.SIGNATURES) == declared_functions()


def test_binding_refuses_to_work_without_the_library(tmp_path, monkeypatch):
    import importlib
    import paged_kv_cache_81_amd._lib as L
    monkeypatch.setenv("PKV_LIBRARY", str(tmp_path / "missing.so"))
    try:
        importlib.reload(L)  # importing works (the build script needs that) ...
        with pytest.raises(ImportError):
            L.lib.pkv_last_error()  # ... but the first call refuses
    finally:
        monkeypatch.delenv("PKV_LIBRARY")
        importlib.reload(L)


@pytest.fixture
def lib():
    from paged_kv_cache_81_amd._lib import lib
    return lib


def test_partition_choice(lib):
    F32, BF16 = 0, 1
    # automatic, bf16: whole sequences when the batch fills the GPU with
    # (sequence, kv-head group) work units in whole rounds of 512 -- 256
    # sequences x 2 groups of 4 kv heads --, in 4 rounds or more, or when a
    # merge would have more than 4096 rows ...
    assert lib.paged_attention_partition_size(256, 32, 8, 128, 16, 1280, 0, BF16) == 1280
    assert lib.paged_attention_partition_size(2000, 8, 2, 64, 16, 100, 0, BF16) == 128
    assert lib.paged_attention_partition_size(256, 40, 40, 128, 16, 2034, 0, BF16) == 2048
    assert lib.paged_attention_partition_size(160, 40, 40, 128, 16, 2034, 0, BF16) == 2048
    # ... else the stream schedule (0): too few units, or 64 sequences x 10
    # groups = 1.25 rounds with a 2560-row merge
    for S, L in ((4, 100), (4, 32768), (4, 0), (8, 2034), (511, 5000)):
        assert lib.paged_attention_partition_size(S, 8, 2, 128, 16, L, 0, BF16) == 0
    assert lib.paged_attention_partition_size(64, 40, 40, 128, 16, 2034, 0, BF16) == 0
    assert lib.paged_attention_partition_size(4, 8, 2, 64, 16, 1000, 0, F32) == 64
    assert lib.paged_attention_partition_size(4, 8, 2, 64, 48, 1000, 0, F32) == 96
    # requests must be whole 32-token steps and whole blocks
    assert lib.paged_attention_partition_size(4, 8, 2, 128, 16, 9999, 96, BF16) == 96
    assert lib.paged_attention_partition_size(4, 8, 2, 128, 64, 9999, 96, BF16) == -1
    assert lib.paged_attention_partition_size(4, 8, 2, 128, 64, 9999, 128, BF16) == 128
    assert lib.paged_attention_partition_size(4, 8, 2, 128, 48, 9999, 96, F32) == 96
    assert lib.paged_attention_partition_size(4, 8, 2, 128, 16, 9999, 1024, F32) == -1
    assert b"multiple" in lib.pkv_last_error()
    assert lib.paged_attention_partition_size(4, 7, 2, 128, 16, 100, 0, BF16) == -1


def test_workspace_bytes(lib):
    BF16 = 1
    assert lib.paged_attention_workspace_bytes(16, 64, 8, 128, 32, 512, 512, BF16) == 0
    S, Hq, D, L, P = 16, 64, 128, 32768, 512
    rows = S * Hq * (L // P)
    want = (rows * D * 4 + 255) // 256 * 256 + rows * 8
    assert lib.paged_attention_workspace_bytes(S, Hq, 8, D, 32, L, P, BF16) == want


def test_host_checks_reject_bad_arguments(lib):
    p = ctypes.c_void_p(0x1000)  # never dereferenced: the checks fail first
    BF16 = 1
    args = dict(out=p, out_dtype=0, query=p, kv=p, tables=p, width=4, lens=p, S=2, Hq=8, Hkv=2,
                D=128, B=16, NB=10, scale=0.1, max_len=64, P=0, ws=None, ws_bytes=0, dtype=BF16,
                flags=0, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return lib.paged_attention_decode(a["out"], a["out_dtype"], a["query"], a["kv"], a["tables"],
                                          a["width"], a["lens"], a["S"], a["Hq"], a["Hkv"], a["D"],
                                          a["B"], a["NB"], a["scale"], a["max_len"], a["P"], a["ws"],
                                          a["ws_bytes"], a["dtype"], a["flags"], a["stream"])
    assert call(D=96) == -2
    assert call(B=12) == -2                     # bf16 blocks of 12 are not built
    assert call(Hq=7) == -1
    assert call(query=None) == -1
    assert call(out=ctypes.c_void_p(0x1004)) == -1   # misaligned
    assert call(P=48) == -1
    assert call(scale=float("nan")) == -1
    assert call(max_len=4096, P=512) == -3      # needs a workspace
    assert call(flags=2) == -1                  # unknown flag
    assert call(S=0) == 0                        # nothing to do
    assert b"workspace" in lib.pkv_last_error() or lib.pkv_last_error() == b""
    assert lib.paged_kv_write(p, p, p, p, 0, 10, 16, 2, 128, BF16, None) == 0
    assert lib.paged_kv_write(p, p, p, p, 4, 10, 16, 2, 4, BF16, None) == -2
    assert lib.paged_kv_write(None, p, p, p, 4, 10, 16, 2, 128, BF16, None) == -1
    assert lib.paged_kv_slot_mapping(p, p, 0, None, p, 4, 4, 16, 10, None) == -1
    assert lib.paged_kv_gather(p, p, p, p, 4, p, 2, 2, 128, 16, 10, 64, 7, None) == -1


def test_prefill_host_checks(lib):
    """Prefill argument checks, made before anything is launched: the bf16
    kernel ranks a launch's work in LDS, which bounds the sequences per call."""
    p = ctypes.c_void_p(0x1000)  # never dereferenced: the checks fail first
    BF16 = 1

    def call(S, D=128, Hq=8, Hkv=2, T=4096, maxq=64):
        return lib.paged_attention_prefill(p, 0, p, p, T, maxq, p, p, 4, p, S, Hq, Hkv, D, 16, 10,
                                           0.1, BF16, None)
    for D, most in ((128, 10914), (64, 5453)):   # the limits the header states
        assert call(most + 1, D=D) == -2
        assert f"at most {most} sequences".encode() in lib.pkv_last_error()
    assert call(1, Hq=7) == -1
    assert call(1, T=1 << 30) == -2             # tokens x 4 heads per kv head overflows
    assert call(0) == 0                          # nothing to do


def test_shared_prefix_host_checks(lib):
    """Argument checks of the shared-prefix decode and the fused write, all
    made before anything is launched."""
    p = ctypes.c_void_p(0x1000)  # never dereferenced: the checks fail first
    F32, BF16 = 0, 1
    args = dict(out=p, out_dtype=0, query=p, kv=p, tables=p, width=4, lens=p, gs=p, pl=p, ng=2,
                S=4, Hq=8, Hkv=2, D=128, B=16, NB=10, scale=0.1, max_len=64, max_prefix=32, P=0,
                ws=p, ws_bytes=1 << 30, dtype=BF16, flags=0, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return lib.paged_attention_decode_shared(
            a["out"], a["out_dtype"], a["query"], a["kv"], a["tables"], a["width"], a["lens"],
            a["gs"], a["pl"], a["ng"], a["S"], a["Hq"], a["Hkv"], a["D"], a["B"], a["NB"],
            a["scale"], a["max_len"], a["max_prefix"], a["P"], a["ws"], a["ws_bytes"], a["dtype"],
            a["flags"], a["stream"])
    assert call(dtype=F32) == -2                # bf16 only
    assert call(D=96) == -2
    assert call(B=12) == -2
    assert call(S=600) == -2                    # more than 512 sequences
    assert call(Hq=7) == -1
    assert call(ng=0) == -1 and call(ng=5) == -1   # 1 <= groups <= sequences
    assert call(gs=None) == -1 and call(pl=None) == -1
    assert call(max_prefix=-1) == -1
    assert call(P=48) == -1                     # not a multiple of 32
    assert call(ws_bytes=16) == -3
    assert call(flags=2) == -1
    assert call(out=ctypes.c_void_p(0x1004)) == -1
    assert call(S=0) == 0
    # the automatic partition is a multiple of the unit; a request is checked
    assert lib.paged_attention_shared_partition_size(256, 32, 8, 128, 16, 32, 1024, 512) == 512
    assert lib.paged_attention_shared_partition_size(256, 32, 8, 128, 64, 32, 1024, 96) == -1
    assert lib.paged_attention_shared_partition_size(8, 8, 2, 128, 16, 8, 0, 0) == 256
    # workspace: parts = ceil(prefix / P) + ceil(len / P), [parts][S][Hq][D] floats,
    # their (m, l), then int32 [4][S]
    S, Hq, D, L, Lp, P = 8, 8, 128, 1000, 512, 256
    parts = 2 + 4
    up = lambda b: (b + 255) // 256 * 256
    want = up(parts * S * Hq * D * 4) + up(parts * S * Hq * 8) + up(4 * S * 4)
    assert lib.paged_attention_shared_workspace_bytes(S, Hq, 2, D, 16, 2, L, Lp, P) == want

    # the fused slot derivation + write
    assert lib.paged_kv_write_positions(p, p, p, p, 4, None, p, None, 0, 4, 10, 16, 2, 128, BF16,
                                        None) == 0
    assert lib.paged_kv_write_positions(p, p, p, p, 4, None, p, None, 4, 4, 10, 16, 2, 4, BF16,
                                        None) == -2
    assert lib.paged_kv_write_positions(p, p, p, None, 4, None, p, None, 4, 4, 10, 16, 2, 128,
                                        BF16, None) == -1
    assert lib.paged_kv_write_positions(p, p, p, p, 0, None, p, None, 4, 4, 10, 16, 2, 128, BF16,
                                        None) == -1


def test_shared_plan_host_checks(lib):
    """Sizing and argument checks of the shared-prefix plan and the planned
    decode, all made before anything is launched."""
    p = ctypes.c_void_p(0x1000)  # never dereferenced: the checks fail first
    BF16 = 1
    # header of 64 ints, the sequences' records [4][S] padded to 64 ints, then
    # 72 ints per item; items at most: (kv-head groups) x (column blocks
    # S*G/16 + groups) x prefix parts + S x (kv-head groups) x (head chunks)
    # x parts of the longest sequence -- here 1 x (2 + 2) x 2 + 8 x 1 x 1 x 4
    S, Hq, Hkv, B, ng, L, Lp, P = 8, 8, 2, 16, 2, 1000, 512, 256
    items = 1 * (2 + 2) * 2 + 8 * 1 * 1 * 4
    want = (64 + 64 + items * 72) * 4
    assert lib.paged_attention_shared_plan_bytes(S, Hq, Hkv, B, ng, L, Lp, P) == want
    assert lib.paged_attention_shared_plan_bytes(S, Hq, Hkv, B, ng, L, Lp, 48) == 0
    assert lib.paged_attention_shared_plan_bytes(S, Hq, Hkv, B, 0, L, Lp, P) == 0

    pa = dict(plan=p, plan_bytes=1 << 30, tables=p, width=4, lens=p, gs=p, pl=p, ng=2, S=4, Hq=8,
              Hkv=2, B=16, max_len=64, max_prefix=32, P=0, stream=None)

    def plan(**kw):
        a = dict(pa, **kw)
        return lib.paged_attention_shared_plan(
            a["plan"], a["plan_bytes"], a["tables"], a["width"], a["lens"], a["gs"], a["pl"],
            a["ng"], a["S"], a["Hq"], a["Hkv"], a["B"], a["max_len"], a["max_prefix"], a["P"],
            a["stream"])
    assert plan(plan=None) == -1 and plan(gs=None) == -1
    assert plan(plan=ctypes.c_void_p(0x1010)) == -1   # 256-byte alignment
    assert plan(plan_bytes=64) == -3
    assert plan(B=12) == -2 and plan(S=600) == -2
    assert plan(ng=0) == -1 and plan(ng=5) == -1
    assert plan(P=48) == -1 and plan(max_prefix=-1) == -1 and plan(Hq=7) == -1
    assert plan(S=0) == 0

    args = [p, 0, p, p, p, 4, p, p, p, 2, 4, 8, 2, 128, 16, 10, 0.1, 64, 32, 0, p, 1 << 30, BF16, 0]
    for fn in (lib.paged_attention_decode_shared_planned,
               lib.paged_attention_shared_planned_partitions,
               lib.paged_attention_shared_planned_merge):
        assert fn(*args, None, 1 << 30, None) == -1              # no plan
        assert fn(*args, ctypes.c_void_p(0x1010), 1 << 30, None) == -1
        assert fn(*args, p, 64, None) == -3                      # plan too small
        assert fn(*(args[:10] + [0] + args[11:]), p, 64, None) == 0  # no sequences


def test_decode_append_host_checks(lib):
    """Argument checks of the decode step with its write, made before
    anything is launched (the new tokens' key and value must both be given
    and 16-byte aligned; the rest is checked as for the plain decode)."""
    p = ctypes.c_void_p(0x1000)  # never dereferenced: the checks fail first
    args = dict(out=p, out_dtype=0, query=p, key=p, value=p, kv=p, tables=p, width=4, lens=p,
                S=4, Hq=8, Hkv=2, D=128, B=16, NB=10, scale=0.1, max_len=64, P=0, ws=p,
                ws_bytes=1 << 30, dtype=1, flags=0, stream=None)

    def call(fn, **kw):
        a = dict(args, **kw)
        return fn(a["out"], a["out_dtype"], a["query"], a["key"], a["value"], a["kv"], a["tables"],
                  a["width"], a["lens"], a["S"], a["Hq"], a["Hkv"], a["D"], a["B"], a["NB"],
                  a["scale"], a["max_len"], a["P"], a["ws"], a["ws_bytes"], a["dtype"], a["flags"],
                  a["stream"])
    for fn in (lib.paged_attention_decode_append, lib.paged_attention_append_partitions):
        assert call(fn, value=None) == -1
        assert call(fn, key=None) == -1
        assert call(fn, key=ctypes.c_void_p(0x1008)) == -1     # misaligned
        assert call(fn, value=ctypes.c_void_p(0x1004)) == -1
        assert call(fn, D=96) == -2
        assert call(fn, Hq=7) == -1
        assert call(fn, flags=4) == -1
        assert call(fn, S=0) == 0
    # where the write goes: only the stream schedule (bf16, automatic
    # partitioning) can store it inside the attention launch
    assert lib.paged_attention_append_in_launch(4, 7, 2, 128, 16, 64, 0, 1) == -1
    assert lib.paged_attention_append_in_launch(4, 8, 2, 128, 16, 64, 0, 0) == 1   # fp32: in launch
    assert lib.paged_attention_append_in_launch(4, 8, 2, 128, 16, 64, 64, 1) == 0  # fixed


def test_split_calls_need_their_buffers():
    """The two launches of a split decode share out and workspace, so the
    binding refuses to make fresh ones for either call (a fresh workspace
    would leave the merge reading memory nobody wrote)."""
    import torch

    import paged_kv_cache_81_amd as pkv
    q = torch.zeros((2, 8, 64), dtype=torch.bfloat16)
    kv = torch.zeros((2, 4, 16, 2, 64), dtype=torch.bfloat16)
    tables = torch.zeros((2, 4), dtype=torch.int32)
    lens = torch.ones(2, dtype=torch.int32)
    ws = torch.zeros(256, dtype=torch.uint8)
    out = torch.zeros((2, 8, 64), dtype=torch.float32)
    for fn in (pkv.attention_partitions, pkv.attention_merge):
        with pytest.raises(ValueError, match="out="):
            fn(q, kv, tables, lens, 0.125, 16, workspace=ws)
        with pytest.raises(ValueError, match="workspace="):
            fn(q, kv, tables, lens, 0.125, 16, out=out)
    with pytest.raises(ValueError, match="workspace="):
        pkv.attention_append_partitions(q, q[:, :2], q[:, :2], kv, tables, lens, 0.125, 16,
                                        out=out)
