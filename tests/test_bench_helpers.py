"""Host-side helpers of bench.py (no GPU): the source hash that ties the
committed counter summary to the kernels, and the lookup that refuses a
summary taken on other sources, another block size or another kernel."""
import json
import os

import bench


def test_source_hash_covers_every_attention_kernel_source():
    names = {os.path.basename(p) for p in bench.KERNEL_SOURCES}
    for f in ("api.hip", "attention_bf16.hip", "attention_bf16_stream.hip",
              "attention_bf16_shared.hip", "attention_bf16_wave.hpp", "attention_f32.hip",
              "common.hpp"):
        assert f in names, f
    assert "prefill.hip" in {os.path.basename(p) for p in bench.PREFILL_SOURCES}
    assert bench.kernel_source_sha() != bench.kernel_source_sha(bench.PREFILL_SOURCES)


def test_traffic_lookup_checks_source_block_size_and_kernel(tmp_path, monkeypatch):
    table = {"w": {"kernel": "void pkv::attention_bf16_stream_kernel<64, 16, 2, true, false>(x)",
                   "kernel_source_sha": "a" * 16, "block_size": 16,
                   "hbm_bytes_per_launch": 123}}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "attention_traffic.json").write_text(json.dumps(table))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda sources=None: "a" * 16)
    assert bench.measured_traffic("w", 16, "attention_bf16_stream_kernel<64,16>") == 123
    assert bench.measured_traffic("w", 32, "attention_bf16_stream_kernel<64,16>") is None
    assert bench.measured_traffic("w", 16, "attention_bf16_kernel<64,16>") is None
    assert bench.measured_traffic("other", 16) is None
    table["w"]["kernel_source_sha"] = "0" * 16
    (prof / "attention_traffic.json").write_text(json.dumps(table))
    assert bench.measured_traffic("w", 16) is None
