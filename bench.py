#!/usr/bin/env python3
"""One-GPU benchmark of the paged decode step.

A step is one pass of the whole hot path over one batch for one attention
layer: the slot of each sequence's new token (slot mapping) and the KV write,
the attention pass over the paged cache and the log-sum-exp merge of context
partitions.  The write goes into the attention launch
(paged_attention_append_partitions) where every sequence appends a token;
otherwise, or with ``--separate-write``, it is a launch of its own
(paged_kv_write_positions).  A model has many layers, each with its own cache pool indexed by
the same block tables; consecutive steps here cycle through ``--layers`` such
pools, as the layers of a decode step do, so no step finds its K/V still in a
cache from the previous one.  Inputs are resident in HBM before timing starts;
the K timed steps are captured in one HIP graph and replayed once.

Prints one JSON line for the headline workload (``--workload``, default the
OPT-13B-shaped batch).  ``value`` is the KV-read throughput of the step: the
bytes the queries read through their block tables (sum over sequences of
L * 2 * num_kv_heads * head_size * element bytes) divided by the step time.
``roofline`` relates the attention kernel alone (its average launch duration:
HIP events on the launch stream around a graph of consecutive launches) to
the MI355X HBM peak; ``*_dist`` give p10/p50/p90 over repeated replays;
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload on one thread and (``all_cores``) on the host's cores, naming the
CPU; ``block_ops`` times the copy-on-write and swap block copies at the
workload's block geometry.  ``ceiling`` is the streaming-read rate of a
plain read kernel (pkv_read_ceiling) over 2 GiB and at the headline's bytes
per launch, and ``frac_of_ceiling`` the attention kernel's share of the
latter.  ``configs`` holds the same figures (step, kernels, roofline,
size-matched ceiling, CPU baselines) for all five decode workloads.

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--only] [--layers N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attn µs/step + KV-read GB/s (% of MI355X HBM peak)"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
# GPU clock cycles of the spin queued before each separately timed launch
# (tens of microseconds: longer than the host takes to queue the launch)
SPIN_CYCLES = 100_000
DEFAULT_WORKLOAD = "opt13b_mha"
# layer caches the steps cycle through: the model's depth where the workload
# is a model's layer shape (OPT-13B 40, Qwen2-0.5B 24), else enough pools to
# hold several times the 256 MB memory-side cache
DEFAULT_LAYERS = {"opt13b_mha": 40, "qwen2_gqa": 24, "shared_prefix": 8, "long_context": 4,
                  "tiny": 1, "prefill_opt13b": 40, "prefill_qwen2": 24}
# the sources that decide what the attention launch does (the counter
# summary in profiles/ holds for this set only)
KERNEL_SOURCES = ["paged_kv_cache_81_amd/csrc/api.hip",
                  "paged_kv_cache_81_amd/csrc/attention_bf16.hip",
                  "paged_kv_cache_81_amd/csrc/attention_bf16_stream.hip",
                  "paged_kv_cache_81_amd/csrc/attention_bf16_shared.hip",
                  "paged_kv_cache_81_amd/csrc/attention_bf16_wave.hpp",
                  "paged_kv_cache_81_amd/csrc/attention_f32.hip",
                  "paged_kv_cache_81_amd/csrc/common.hpp"]
# ... and the prefill launch
PREFILL_SOURCES = ["paged_kv_cache_81_amd/csrc/api.hip",
                   "paged_kv_cache_81_amd/csrc/prefill.hip",
                   "paged_kv_cache_81_amd/csrc/attention_bf16_wave.hpp",
                   "paged_kv_cache_81_amd/csrc/common.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(sources=None) -> str:
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kv_bytes(w) -> int:
    """K/V bytes the queries read through their tables (logical)."""
    import numpy as np
    return int(w.context_lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_size * w.elem_bytes


def unique_kv_bytes(w) -> int:
    """K/V bytes of the distinct cache rows the batch reads (a block shared by
    several sequences counts once): every cached row plus each appended token."""
    import numpy as np
    rows = w.cached_k.shape[0] + int(np.count_nonzero(w.new_pos >= 0))
    return rows * 2 * w.num_kv_heads * w.head_size * w.elem_bytes


def _is_prefill(workload: str) -> bool:
    return workload.startswith("prefill_")


def measured_traffic(workload: str, block_size=None, kernel=None):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source and block size (and
    on the kernel named, e.g. "attention_bf16_stream_kernel<128,16>"); else
    None."""
    path = os.path.join(ROOT, "profiles", "attention_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    sources = PREFILL_SOURCES if _is_prefill(workload) else KERNEL_SOURCES
    if not rec or rec.get("kernel_source_sha") != kernel_source_sha(sources):
        return None
    if block_size is not None and rec.get("block_size", block_size) != block_size:
        return None
    if kernel is not None and kernel.split("<")[0] + "<" not in rec.get("kernel", ""):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_means(path: str, kernel_part: str, min_value: float = 0.0):
    """Mean Counter_Value (KiB per dispatch) of the dispatches whose kernel
    name contains kernel_part (and whose value is at least min_value)."""
    import csv
    vals, name = [], None
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_part in r["Kernel_Name"] and float(r["Counter_Value"]) >= min_value:
                vals.append(float(r["Counter_Value"]))
                name = r["Kernel_Name"]
    if not vals:
        raise SystemExit(f"no dispatch of {kernel_part!r} in {path}")
    return sum(vals) / len(vals), len(vals), name


def summarize_counters(d: str, workload: str) -> int:
    """HBM bytes per attention launch from rocprofv3 counter passes, scaled
    by what the same counters read for a 1 GiB copy."""
    import workloads

    csv_of = lambda c: os.path.join(d, c, "run_counter_collection.csv")
    part = ("prefill_bf16" if _is_prefill(workload) else
            "attention_f32" if workload == "tiny" else "attention_bf16")
    fetch, n, kname = _counter_means(csv_of("FETCH_SIZE"), part)
    write, _, _ = _counter_means(csv_of("WRITE_SIZE"), part)
    # the 1 GiB copies (smaller copies of the same kernel in the run are ignored)
    cfetch, _, _ = _counter_means(csv_of("cal_FETCH_SIZE"), "copyBuffer", 1e5)
    cwrite, _, _ = _counter_means(csv_of("cal_WRITE_SIZE"), "copyBuffer", 1e5)
    fscale, wscale = (1 << 30) / (cfetch * 1024), (1 << 30) / (cwrite * 1024)
    if _is_prefill(workload):
        w = workloads.PREFILL[workload]().cache
        sources = PREFILL_SOURCES
    else:
        w = workloads.make(workload)
        sources = KERNEL_SOURCES
    rec = {
        "kernel": kname,
        "kernel_source_sha": kernel_source_sha(sources),
        "block_size": w.block_size,
        "fetch_size_kib_per_launch": round(fetch, 2),
        "write_size_kib_per_launch": round(write, 2),
        "copy_fetch_size_kib": round(cfetch, 3),
        "copy_write_size_kib": round(cwrite, 3),
        "fetch_scale": round(fscale, 6),
        "write_scale": round(wscale, 6),
        "hbm_read_bytes_per_launch": round(fetch * 1024 * fscale),
        "hbm_write_bytes_per_launch": round(write * 1024 * wscale),
        "hbm_bytes_per_launch": round(fetch * 1024 * fscale + write * 1024 * wscale),
        "algorithmic_kv_bytes_per_launch": unique_kv_bytes(w),
        "logical_kv_bytes_per_launch": kv_bytes(w),
        "launches_counted": n,
    }
    path = os.path.join(ROOT, "profiles", "attention_traffic.json")
    table = json.load(open(path)) if os.path.exists(path) else {}
    table[workload] = rec
    with open(path, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))
    return 0


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_share() -> int:
    """Host cores this process may use: its CPU affinity, at most 16 (the
    share of one GPU on a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# state the forked CPU-baseline workers read (set before they are forked)
_CPU_JOB = {}


def _oracle_step(s: int) -> int:
    """One sequence's decode step through the oracle, as it is: slot mapping
    and write of the new token (idempotent; sequences write disjoint slots),
    gather through the table, float64 attention.  Returns the KV bytes read."""
    import numpy as np

    import oracle
    w, pool, per_tok = _CPU_JOB["w"], _CPU_JOB["pool"], _CPU_JOB["per_tok"]
    slot = oracle.slot_mapping_ref(w.block_tables, np.array([s]), w.new_pos[s:s + 1], w.block_size)
    oracle.write_ref(pool, w.new_k[s:s + 1], w.new_v[s:s + 1], slot)
    L = int(w.context_lens[s])
    k, v = oracle.gather_ref(pool, w.block_tables[s], L)
    oracle.attention_ref(oracle.to_f64(w.query[s], w.dtype), oracle.to_f64(k, w.dtype),
                         oracle.to_f64(v, w.dtype), w.scale)
    return L * per_tok


def _oracle_worker(args):
    """A forked worker: sequences first, first + stride, ... of the batch,
    repeated, until `seconds` have passed; (bytes, steps, seconds)."""
    from threadpoolctl import threadpool_limits
    first, stride, seconds = args
    n_seq = _CPU_JOB["w"].num_seqs
    done = n = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        s = first
        while time.perf_counter() - t0 < seconds:
            done += _oracle_step(s % n_seq)
            n += 1
            s += stride
        dt = time.perf_counter() - t0
    return done, n, dt


def cpu_baseline(w, seconds: float, processes: int = 1) -> dict:
    """The CPU oracle on a bounded sample of the workload's sequences: per
    sequence, slot mapping + write of the new token, gather through the
    table, float64 attention -- the oracle's functions as they are, one
    sequence at a time (numpy's own thread pool held to one thread), passes
    over the batch repeated for about ``seconds``; with ``processes`` > 1,
    that many forked processes take every processes-th sequence each.  Call
    it before the GPU is initialised (the workers are forked)."""
    import multiprocessing
    from threadpoolctl import threadpool_limits

    import oracle
    from tests import gpu_harness as H

    with threadpool_limits(limits=1):
        pool = H.nan_pool_numpy(w)
        oracle.write_ref(pool, w.cached_k, w.cached_v,
                         oracle.slot_mapping_ref(w.block_tables, w.cached_seq, w.cached_pos,
                                                 w.block_size))
    _CPU_JOB.update(w=w, pool=pool, per_tok=2 * w.num_kv_heads * w.head_size * w.elem_bytes)
    if processes <= 1:
        done, n, dt = _oracle_worker((0, 1, seconds))
    else:
        with multiprocessing.get_context("fork").Pool(processes) as mp:
            parts = mp.map(_oracle_worker, [(i, processes, seconds) for i in range(processes)])
        done = sum(p[0] for p in parts)
        n = sum(p[1] for p in parts)
        dt = max(p[2] for p in parts)
    step_bytes = int(w.context_lens.sum()) * _CPU_JOB["per_tok"]
    _CPU_JOB.clear()
    return {"value": round(done / dt / 1e9, 4), "unit": "GB/s", "cores": processes,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{n} sequence decode steps of {w.name} ({n / w.num_seqs:.2f} passes over "
                      f"its {w.num_seqs} sequences, {done / 1e6:.1f} MB of KV), float64 numpy, "
                      + (f"{processes} processes" if processes > 1 else "one thread")
                      + f", {dt:.1f} s",
            "us_per_step_extrapolated": round(step_bytes / (done / dt) * 1e6, 1)}


def block_ops(w, dev, reps: int = 10) -> dict:
    """Copy-on-write and swap copies at the workload's block geometry, each
    one ``paged_kv_copy_blocks`` launch timed with HIP events on its stream:
    one block copied per sequence within a device pool (the copy a forked
    sample makes before its first write into a shared block), and a group of
    blocks swapped to a pinned host pool and back (PCIe).  Caches are cold
    (a 1 GiB read runs before each launch); the copy-on-write copy is also
    timed with warm caches.  Bytes count each
    block's keys and values once read and once written; ``memcpy_GBps`` is a
    plain contiguous device/host copy of the same bytes for comparison."""
    import numpy as np
    import torch

    import paged_kv_cache_81_amd as pkv

    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    geo = (w.block_size, w.num_kv_heads, w.head_size)
    blk = 2 * int(np.prod(geo)) * (2 if w.dtype == "bf16" else 4)
    rng = np.random.default_rng(5)
    cur = torch.cuda.current_stream(dev)

    # work queued before each timed launch keeps the GPU busy while the host
    # prepares the launch, so the events bracket the copy alone: a 1 GiB read
    # (evicts the caches without leaving dirty lines) or a spin (caches warm)
    sweep = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def timed(fn, cold=True):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for i, (a, b) in enumerate(ev):
            if cold:
                sweep.sum()
            else:
                torch.cuda._sleep(400_000)
            a.record(cur)
            fn()
            b.record(cur)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3  # us

    out = {"block_bytes": blk}
    n_dev = 2048
    pool = torch.empty((2, n_dev) + geo, dtype=tdt, device=dev).normal_()
    ids = rng.permutation(n_dev).astype(np.int32)
    n = w.num_seqs
    src = torch.from_numpy(ids[:n]).to(dev)
    dst = torch.from_numpy(ids[n:2 * n]).to(dev)
    us = timed(lambda: pkv.copy_blocks(pool, pool, src, dst))
    us_hot = timed(lambda: pkv.copy_blocks(pool, pool, src, dst), cold=False)
    out["cow_copy"] = {"copies": n, "us": round(us, 2), "GBps": round(2 * n * blk / us / 1e3, 1),
                       "us_warm_caches": round(us_hot, 2)}

    n_swap = 512
    host = torch.empty((2, n_swap) + geo, dtype=tdt, pin_memory=True)
    src = torch.from_numpy(ids[:n_swap]).to(dev)
    hid = torch.arange(n_swap, dtype=torch.int32, device=dev)
    us_out = timed(lambda: pkv.copy_blocks(host, pool, src, hid))
    us_in = timed(lambda: pkv.copy_blocks(pool, host, hid, src))
    flat_dev = torch.empty(n_swap * blk, dtype=torch.uint8, device=dev)
    flat_host = torch.empty(n_swap * blk, dtype=torch.uint8, pin_memory=True)
    us_d2h = timed(lambda: flat_host.copy_(flat_dev, non_blocking=True))
    us_h2d = timed(lambda: flat_dev.copy_(flat_host, non_blocking=True))
    b = n_swap * blk
    out["swap_out"] = {"blocks": n_swap, "us": round(us_out, 1), "GBps": round(b / us_out / 1e3, 1),
                       "memcpy_GBps": round(b / us_d2h / 1e3, 1)}
    out["swap_in"] = {"blocks": n_swap, "us": round(us_in, 1), "GBps": round(b / us_in / 1e3, 1),
                      "memcpy_GBps": round(b / us_h2d / 1e3, 1)}
    return out


PREFILL_METRIC = "paged prefill attn TFLOP/s (% of MI355X bf16 MFMA dense peak)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, AMD's published figure


def prefill_cpu_baseline(pw, seconds: float) -> dict:
    """The CPU oracle, one thread, on a bounded sample of the prefill rows:
    each row is float64 attention over its sequence's keys up to its position."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from tests import gpu_harness as H

    w = pw.cache
    with threadpool_limits(limits=1):
        pool = H.nan_pool_numpy(w)
        oracle.write_ref(pool, w.cached_k, w.cached_v,
                         oracle.slot_mapping_ref(w.block_tables, w.cached_seq, w.cached_pos,
                                                 w.block_size))
        oracle.write_ref(pool, w.new_k, w.new_v,
                         oracle.slot_mapping_ref(w.block_tables, np.arange(w.num_seqs), w.new_pos,
                                                 w.block_size))
        rng = np.random.default_rng(0)
        flops, n = 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            r = int(rng.integers(0, pw.num_tokens))
            s = int(np.searchsorted(pw.query_start, r, side="right") - 1)
            L = int(w.context_lens[s])
            p = int(oracle.chunk_positions(L, int(pw.chunk_lens[s]))[r - pw.query_start[s]])
            k, v = oracle.gather_ref(pool, w.block_tables[s], p + 1)
            oracle.attention_ref(oracle.to_f64(pw.query[r], w.dtype), oracle.to_f64(k, w.dtype),
                                 oracle.to_f64(v, w.dtype), w.scale)
            flops += 4 * w.head_size * w.num_q_heads * (p + 1)
            n += 1
        dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} random query rows of {pw.name} (all heads), float64 numpy, one "
                      f"thread, {dt:.1f} s"}


def prefill_bench(args, dev) -> dict:
    """One step = slot mapping and write of the chunks' K/V, then prefill
    attention, cycling through layer pools; K steps in one graph."""
    import numpy as np
    import torch

    import paged_kv_cache_81_amd._lib as lib_mod
    import workloads
    from paged_kv_cache_81_amd._lib import check, lib
    from tests import gpu_harness as H

    pw = workloads.PREFILL[args.workload](**_block_kw(args))
    w = pw.cache
    S, B, NB = w.num_seqs, w.block_size, w.num_blocks
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_size
    T = pw.num_tokens
    log(f"[bench] workload {pw.name}: S={S} T={T} Hq={Hq} Hkv={Hkv} D={D} B={B} NB={NB} "
        f"sumL={int(w.context_lens.sum())} flops={pw.flops() / 1e9:.1f} G")
    st = H.upload(w, device=dev)
    # the chunks' K/V rows and positions (the last chunk_len tokens of each sequence)
    ks, vs, seqs, poss = [], [], [], []
    for si in range(S):
        k, v = w.logical_kv(si)
        c = int(pw.chunk_lens[si])
        L = int(w.context_lens[si])
        ks.append(k[L - c:])
        vs.append(v[L - c:])
        seqs.append(np.full(c, si, dtype=np.int32))
        poss.append(np.arange(L - c, L, dtype=np.int32))
    ck = H.to_torch(np.concatenate(ks), w.dtype, dev)
    cv = H.to_torch(np.concatenate(vs), w.dtype, dev)
    cseq = torch.from_numpy(np.concatenate(seqs)).to(dev)
    cpos = torch.from_numpy(np.concatenate(poss)).to(dev)
    cslots = torch.empty(T, dtype=torch.int64, device=dev)
    q = H.to_torch(pw.query, w.dtype, dev)
    qs = torch.from_numpy(pw.query_start).to(dev)
    out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    dt = lib_mod.PKV_BF16 if w.dtype == "bf16" else lib_mod.PKV_F32
    nl = args.layers if args.layers is not None else DEFAULT_LAYERS.get(pw.name, 4)
    free, _ = torch.cuda.mem_get_info(dev)
    nl = max(1, min(nl, int(0.5 * free // st.kv.numel() // st.kv.element_size())))
    pools = [st.kv] + [st.kv.clone() for _ in range(nl - 1)]
    torch.cuda.synchronize()

    def calls(sh, layer):
        kv = pools[layer]
        return {
            "kv_write": lambda: check(lib.paged_kv_write_positions(
                ck.data_ptr(), cv.data_ptr(), kv.data_ptr(), st.tables.data_ptr(), w.table_width,
                cseq.data_ptr(), cpos.data_ptr(), cslots.data_ptr(), T, S, NB, B, Hkv, D, dt, sh),
                "kv write"),
            "prefill": lambda: check(lib.paged_attention_prefill(
                out.data_ptr(), 0, q.data_ptr(), qs.data_ptr(), T, pw.max_query_len,
                kv.data_ptr(), st.tables.data_ptr(), w.table_width, st.lens.data_ptr(), S, Hq,
                Hkv, D, B, NB, w.scale, dt, sh), "prefill"),
        }

    cur = torch.cuda.current_stream(dev)
    eager = [calls(cur.cuda_stream, layer) for layer in range(nl)]
    for f in eager[0].values():
        f()
    torch.cuda.synchronize()
    ref_out = out.clone()
    for i in range(args.warmup):
        for f in eager[i % nl].values():
            f()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(cur)
    with torch.cuda.stream(cap):
        captured = [calls(cap.cuda_stream, layer) for layer in range(nl)]
        for f in captured[0].values():
            f()
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                for f in captured[i % nl].values():
                    f()
    cur.wait_stream(cap)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(cur)
    graph.replay()
    t1.record(cur)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step")
    for f in eager[(args.steps - 1) % nl].values():
        f()
    torch.cuda.synchronize()
    if not torch.equal(out, ref_out):
        raise SystemExit("[bench] the timed steps' output differs from the first eager step's")
    # the prefill kernel alone: events around a graph of `reps` consecutive
    # launches (cycling the layer pools), divided by `reps`
    reps = max(10, min(args.steps, 50))
    g = torch.cuda.CUDAGraph()
    cap2 = torch.cuda.Stream(device=dev)
    cap2.wait_stream(cur)
    with torch.cuda.stream(cap2):
        fs = [calls(cap2.cuda_stream, layer)["prefill"] for layer in range(nl)]
        fs[0]()
        cap2.synchronize()
        with torch.cuda.graph(g, stream=cap2):
            for r in range(reps):
                fs[r % nl]()
    cur.wait_stream(cap2)
    torch.cuda.synchronize()
    g.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(cur)
    g.replay()
    b.record(cur)
    torch.cuda.synchronize()
    kernel_us = a.elapsed_time(b) * 1e3 / reps
    flops = pw.flops()
    tflops = flops / (kernel_us * 1e-6) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] prefill kernel {kernel_us:.1f} us = {tflops:.1f} TFLOP/s")
    return {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "accumulate": "f32",
        "data": "synthetic (seeded N(0,1) K/V/q, shuffled block pool)",
        "config": {
            "workload": pw.name, "num_seqs": S, "num_tokens": T, "num_q_heads": Hq,
            "num_kv_heads": Hkv, "head_size": D, "block_size": B, "num_blocks": NB,
            "sum_context_len": int(w.context_lens.sum()), "max_query_len": pw.max_query_len,
            "flops": flops, "graph": True, "layers_cycled": nl,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(pw.name, B),
            "kernel": f"prefill_bf16_kernel<{D},{B}>" if w.dtype == "bf16" else f"prefill_f32_kernel<{D}>",
            "kernel_us": round(kernel_us, 2),
            "algorithmic_flops": flops,
        },
        "kernel_source_sha": kernel_source_sha(PREFILL_SOURCES),
    }


def _block_kw(args) -> dict:
    return {"block_size": args.block_size} if args.block_size else {}


# the five decode workloads, in the order their shapes are listed
ALL_DECODE = ["tiny", "opt13b_mha", "qwen2_gqa", "shared_prefix", "long_context"]


def _graph_avg_us(dev, fns, reps: int, replays: int = 1):
    """Average launch duration (us) of ``reps`` consecutive launches of the
    callables ``fns[r % len(fns)]`` (each given the capturing stream's
    handle), captured in one HIP graph: HIP events on the launch stream
    around each replay, divided by ``reps``.  One value per replay."""
    import torch
    cur = torch.cuda.current_stream(dev)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(cur)
    with torch.cuda.stream(cap):
        fns[0](cap.cuda_stream)
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            for r in range(reps):
                fns[r % len(fns)](cap.cuda_stream)
    cur.wait_stream(cap)
    torch.cuda.synchronize()
    g.replay()  # untimed
    out = []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(cur)
        g.replay()
        b.record(cur)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) * 1e3 / reps)
    del g
    return out


def _dist(xs) -> dict:
    import numpy as np
    return {"p10": round(float(np.percentile(xs, 10)), 2), "p50": round(float(np.percentile(xs, 50)), 2),
            "p90": round(float(np.percentile(xs, 90)), 2), "samples": len(xs)}


def read_ceiling(dev, nbytes: int) -> dict:
    """Best streaming-read rate (GB/s) of ``pkv_read_ceiling`` over a sweep
    of grids and loads in flight, reading ``nbytes`` per launch: a graph of
    launches cycling distinct buffers (at least 1 GiB in all, so no launch
    finds its bytes in the 256 MB memory-side cache, for sizes from 16 MB)."""
    import torch

    from paged_kv_cache_81_amd._lib import check, lib
    nbytes = max(16, nbytes // 16 * 16)
    # (at most 64 buffers: below ~16 MB a launch is bound by its own start and
    # end, not by where its bytes come from)
    nbuf = min(64, max(2, -(-(1 << 30) // nbytes)))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i % 200 + 1)
            for i in range(nbuf)]
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    reps = max(nbuf, min(100, max(10, (2 << 30) // nbytes)))
    best = None
    for grid in (512, 768, 1024, 1536, 2048, 3072):
        for per in (2, 4):
            fns = [(lambda sh, b=b, grid=grid, per=per: check(
                lib.pkv_read_ceiling(b.data_ptr(), nbytes, grid, per, sink.data_ptr(), sh),
                "read ceiling")) for b in bufs]
            us = min(_graph_avg_us(dev, fns, reps, replays=3))
            gbps = nbytes / (us * 1e-6) / 1e9
            if best is None or gbps > best["GBps"]:
                best = {"GBps": round(gbps, 1), "us": round(us, 2), "grid": grid,
                        "loads_in_flight": per}
    del bufs, sink
    torch.cuda.empty_cache()
    best["bytes"] = nbytes
    return best


def decode_bench(name, args, dev, headline: bool) -> dict:
    """One decode workload: the timed steps (write + attention + merge,
    cycling layer pools, in one graph), each kernel alone, and the
    headline's block copies.  Returns the result line's fields for it."""
    import numpy as np
    import torch

    import paged_kv_cache_81_amd as pkv
    import paged_kv_cache_81_amd._lib as lib_mod
    import workloads
    from paged_kv_cache_81_amd._lib import check, lib
    from tests import gpu_harness as H

    t = time.time()
    w = workloads.make(name, **_block_kw(args))
    log(f"[bench] workload {w.name}: S={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"D={w.head_size} B={w.block_size} NB={w.num_blocks} sumL={int(w.context_lens.sum())} "
        f"(generated in {time.time() - t:.1f} s)")
    st = H.upload(w, device=dev)
    torch.cuda.synchronize()

    S, B, NB = w.num_seqs, w.block_size, w.num_blocks
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_size
    dt = 1 if w.dtype == "bf16" else 0
    tdt = torch.bfloat16 if dt else torch.float32
    P = w.partition_size if args.partition_size is None else args.partition_size
    P = pkv.partition_size(S, Hq, Hkv, D, B, w.max_context_len, P, tdt)
    ws_bytes = pkv.workspace_bytes(S, Hq, Hkv, D, B, w.max_context_len, P, tdt)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    shared = bool(w.meta.get("forks"))  # forks alias their prompt's blocks
    # forks read their shared prompt once per group (the shared-prefix
    # decode) unless told to read it per sequence through the caches
    grouped = shared and not args.no_shared_prefix
    if args.kv_flags == "auto":
        flags = lib_mod.PKV_ATTN_CACHED_KV if shared else 0
    else:
        flags = lib_mod.PKV_ATTN_CACHED_KV if args.kv_flags == "cached" else 0
    if grouped:
        g_starts, g_plens, g_maxp = pkv.prefix_groups(w.block_tables, w.context_lens, B)
        n_groups = len(g_plens)
        d_starts = torch.from_numpy(g_starts).to(dev)
        d_plens = torch.from_numpy(g_plens).to(dev)
        P = lib.paged_attention_shared_partition_size(S, Hq, Hkv, D, B, n_groups, g_maxp,
                                                      args.partition_size or 0)
        ws_bytes = pkv.shared_workspace_bytes(S, Hq, Hkv, D, B, n_groups, w.max_context_len,
                                              g_maxp, P)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        # the work list, made once per decode step (every layer reads the
        # same tables) and read by each layer's launches
        if not args.no_plan:
            plan_bytes = pkv.shared_plan_bytes(S, Hq, Hkv, B, n_groups, w.max_context_len, g_maxp,
                                               P)
            plan_buf = torch.empty(max(plan_bytes, 256), dtype=torch.uint8, device=dev)
        log(f"[bench] shared-prefix decode: {n_groups} groups, longest prefix {g_maxp}, "
            f"partition {P}")

    # the write goes into the attention launch (paged_attention_append_partitions)
    # when every sequence's new token sits at its last position, the library
    # stores it inside that launch for this batch, and the separate launches
    # were not asked for
    fused_write = (not grouped and not args.separate_write and not args.separate_slot_mapping
                   and bool(np.all(w.new_pos == np.where(w.context_lens > 0,
                                                         w.context_lens - 1, -1)))
                   and lib.paged_attention_append_in_launch(S, Hq, Hkv, D, B, w.max_context_len,
                                                            P, dt) == 1)

    # one cache pool per layer, all indexed by the same block tables
    nl = args.layers if args.layers is not None else DEFAULT_LAYERS.get(w.name, 4)
    free, _ = torch.cuda.mem_get_info(dev)
    nl = max(1, min(nl, int(0.6 * free // st.kv.numel() // st.kv.element_size())))
    pools = [st.kv] + [st.kv.clone() for _ in range(nl - 1)]
    torch.cuda.synchronize()
    log(f"[bench] {nl} layer pools of {st.kv.numel() * st.kv.element_size() / 1e9:.2f} GB, "
        f"partition {P}, flags {flags}")

    def calls(stream_handle, layer):
        kv = pools[layer]
        slot_a = (st.new_slots.data_ptr(), st.tables.data_ptr(), w.table_width, None,
                  st.new_pos.data_ptr(), S, S, B, NB, stream_handle)
        write_a = (st.new_k.data_ptr(), st.new_v.data_ptr(), kv.data_ptr(),
                   st.new_slots.data_ptr(), S, NB, B, Hkv, D, dt, stream_handle)
        # slot of each new token and its write in one launch (the slots are
        # recorded too), or the two separate launches
        wpos_a = (st.new_k.data_ptr(), st.new_v.data_ptr(), kv.data_ptr(), st.tables.data_ptr(),
                  w.table_width, None, st.new_pos.data_ptr(), st.new_slots.data_ptr(), S, S, NB, B,
                  Hkv, D, dt, stream_handle)
        if args.separate_slot_mapping:
            write_step = {
                "slot_mapping": lambda: check(lib.paged_kv_slot_mapping(*slot_a), "slot mapping"),
                "kv_write": lambda: check(lib.paged_kv_write(*write_a), "kv write"),
            }
        else:
            write_step = {
                "kv_write": lambda: check(lib.paged_kv_write_positions(*wpos_a), "kv write"),
            }
        if grouped:
            sh_a = (out.data_ptr(), 0, st.query.data_ptr(), kv.data_ptr(), st.tables.data_ptr(),
                    w.table_width, st.lens.data_ptr(), d_starts.data_ptr(), d_plens.data_ptr(),
                    n_groups, S, Hq, Hkv, D, B, NB, w.scale, w.max_context_len, g_maxp, P,
                    ws.data_ptr(), ws.numel(), dt, flags, stream_handle)
            if not args.no_plan:
                # the plan on the first layer's step: once per nl layer steps
                pl_a = sh_a[:-1] + (plan_buf.data_ptr(), plan_buf.numel(), stream_handle)
                mk_a = (plan_buf.data_ptr(), plan_buf.numel(), st.tables.data_ptr(),
                        w.table_width, st.lens.data_ptr(), d_starts.data_ptr(),
                        d_plens.data_ptr(), n_groups, S, Hq, Hkv, B, w.max_context_len, g_maxp,
                        P, stream_handle)
                plan_step = ({"plan": lambda: check(lib.paged_attention_shared_plan(*mk_a),
                                                    "plan")} if layer == 0 else {})
                return {
                    **plan_step,
                    **write_step,
                    "attention": lambda: check(
                        lib.paged_attention_shared_planned_partitions(*pl_a), "attention"),
                    "merge": lambda: check(lib.paged_attention_shared_planned_merge(*pl_a),
                                           "merge"),
                }
            return {
                **write_step,
                "attention": lambda: check(lib.paged_attention_shared_partitions(*sh_a),
                                           "attention"),
                "merge": lambda: check(lib.paged_attention_shared_merge(*sh_a), "merge"),
            }
        attn_a = (out.data_ptr(), 0, st.query.data_ptr(), kv.data_ptr(), st.tables.data_ptr(),
                  w.table_width, st.lens.data_ptr(), S, Hq, Hkv, D, B, NB, w.scale,
                  w.max_context_len, P, ws.data_ptr(), ws.numel(), dt, flags, stream_handle)
        if fused_write:
            # each sequence's new token is written by the attention launch itself
            app_a = attn_a[:3] + (st.new_k.data_ptr(), st.new_v.data_ptr()) + attn_a[3:]
            return {
                "attention": lambda: check(lib.paged_attention_append_partitions(*app_a),
                                           "attention (with the write)"),
                "merge": lambda: check(lib.paged_attention_merge(*attn_a), "merge"),
            }
        return {
            **write_step,
            "attention": lambda: check(lib.paged_attention_partitions(*attn_a), "attention"),
            "merge": lambda: check(lib.paged_attention_merge(*attn_a), "merge"),
        }

    cur = torch.cuda.current_stream(dev)
    eager = [calls(cur.cuda_stream, layer) for layer in range(nl)]

    def eager_step(i):
        for f in eager[i % nl].values():
            f()

    eager_step(0)
    torch.cuda.synchronize()
    ref_out = out.clone()
    for i in range(args.warmup):
        eager_step(i)
    torch.cuda.synchronize()

    if args.no_graph:
        def run_steps():
            for i in range(args.steps):
                eager_step(i)
    else:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(device=dev)
        cap.wait_stream(cur)
        with torch.cuda.stream(cap):
            captured = [calls(cap.cuda_stream, layer) for layer in range(nl)]
            for f in captured[0].values():
                f()
            cap.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                for i in range(args.steps):
                    for f in captured[i % nl].values():
                        f()
        cur.wait_stream(cap)
        torch.cuda.synchronize()
        run_steps = graph.replay
        run_steps()  # one untimed replay
        torch.cuda.synchronize()

    # exactly K steps between two synchronisations: the step time
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(cur)
    run_steps()
    t1.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    log(f"[bench] {w.name}: {args.steps} steps: {ms_per_step * 1e3:.1f} us/step "
        f"(wall {wall / args.steps * 1e6:.1f} us)")
    # the same replay a few more times, for the spread of the step time
    step_us = [ms_per_step * 1e3]
    for _ in range(args.spread_replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(cur)
        run_steps()
        b.record(cur)
        torch.cuda.synchronize()
        step_us.append(a.elapsed_time(b) * 1e3 / args.steps)
    eager_step((args.steps - 1) % nl if nl > 1 else 0)
    torch.cuda.synchronize()
    if not torch.equal(out, ref_out):
        raise SystemExit(f"[bench] {w.name}: the timed steps' output differs from the first "
                         "eager step's")

    # each kernel on its own, `reps` launches in a row cycling through the
    # layer pools: HIP events on the launch stream around one replay of a
    # graph holding those launches, divided by `reps` -- the kernel's average
    # launch duration, as a kernel trace reports it (event pairs around
    # single launches add the events' own few microseconds to each); the
    # graph is replayed several times for the spread.  With --flush: eager
    # launches, each after a cache-evicting fill and a spin that keeps the
    # GPU busy while the host queues the event pair.
    reps = max(10, min(args.steps, 100))
    names = list(eager[0])
    kernel_us, kernel_dist = {}, {}
    if args.flush:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps * len(names))]
        per = {k: [] for k in names}
        i = 0
        for r in range(reps):
            for kname_, f in eager[r % nl].items():
                flush.fill_(r & 0xFF)
                torch.cuda._sleep(SPIN_CYCLES)
                ev[i][0].record(cur)
                f()
                ev[i][1].record(cur)
                per[kname_].append(i)
                i += 1
        torch.cuda.synchronize()
        for k, idx in per.items():
            xs = [ev[j][0].elapsed_time(ev[j][1]) * 1e3 for j in idx]
            kernel_us[k] = float(np.mean(xs))
            kernel_dist[k] = _dist(xs)
        del flush
    else:
        for kname_ in names:
            # (the plan is only in the first layer's step)
            fns = [(lambda sh, layer=layer, kname_=kname_: calls(sh, layer)[kname_]())
                   for layer in range(nl) if kname_ in eager[layer]]
            xs = _graph_avg_us(dev, fns, reps, replays=1 + args.spread_replays)
            kernel_us[kname_] = xs[0]
            kernel_dist[kname_] = _dist(xs)
    log(f"[bench] {w.name}: per-kernel us: " +
        ", ".join(f"{k} {v:.1f}" for k, v in kernel_us.items()))

    kvb = kv_bytes(w)
    ukvb = unique_kv_bytes(w)
    value = kvb / (ms_per_step * 1e-3) / 1e9
    # the roofline counts each distinct cache row once: reads of blocks shared
    # by several sequences can hit in the caches, and a logical rate above the
    # HBM peak would not be a fraction of it
    attn_gbps = ukvb / (kernel_us["attention"] * 1e-6) / 1e9
    kname = (f"attention_f32_kernel<{D}>" if not dt else
             f"attention_bf16_shared_kernel<{D},{B}>" if grouped else
             f"attention_bf16_stream_kernel<{D},{B}>" if P == 0 else f"attention_bf16_kernel<{D},{B}>")
    traffic = measured_traffic(w.name, B, kname)

    result = {
        "value": round(value, 2),
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_dist": _dist(step_us),
        "hbm_frac_step": round(value / PEAK_HBM_GBPS, 4),
        "dtype": "bf16" if dt else "f32",
        "config": {
            "workload": w.name, "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_size": D, "block_size": B, "num_blocks": NB,
            "sum_context_len": int(w.context_lens.sum()), "max_context_len": w.max_context_len,
            "kv_read_bytes": kvb, "kv_unique_bytes": ukvb, "partition_size": P,
            "reserved_slot_waste": round(float(
                (np.ceil(w.context_lens / B) * B - w.context_lens).sum() /
                max(1, int(w.context_lens.sum()))), 5),
            "table_bytes": int(np.ceil(w.context_lens / B).sum()) * 4,
            "graph": not args.no_graph,
            "layers_cycled": nl,
            "kv_flags": "cached" if flags & lib_mod.PKV_ATTN_CACHED_KV else "streamed",
            "attention_path": ("shared prefix (groups read their prompt once)" if grouped else
                               "per sequence"),
            "kv_write": ("inside the attention launch" if fused_write else
                         "separate launch" + ("es" if args.separate_slot_mapping else "")),
            **({"groups": n_groups, "max_prefix_len": g_maxp,
                "work_list": ("none: each attention launch derives it" if args.no_plan else
                              f"one plan launch per {nl} layer steps (a decode step of an "
                              f"{nl}-layer model), read by every layer's launches")}
               if grouped else {}),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(attn_gbps, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(attn_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel": kname,
            "kernel_us": round(kernel_us["attention"], 2),
            "timing": (f"HIP events around single launches" if args.flush else
                       f"HIP events around a graph of {reps} consecutive launches"),
            "algorithmic_bytes": ukvb,
            "logical_bytes": kvb,
            "logical_GBps": round(kvb / (kernel_us["attention"] * 1e-6) / 1e9, 2),
            "caches": ("evicted before each launch" if args.flush else
                       f"cold: launches cycle through {nl} layer pools" if nl > 1 else "warm"),
        },
        "kernel_us": {k: round(v, 2) for k, v in kernel_us.items()},
        "kernel_us_dist": {**kernel_dist,
                           "what": ("per-launch average over each of several replays of the "
                                    f"graph of {reps} launches" if not args.flush else
                                    "single launches")},
    }
    if headline and not args.no_block_ops:
        result["block_ops"] = block_ops(w, dev)
        log(f"[bench] block ops: {result['block_ops']}")
    del pools, st, ws, out, eager
    if not args.no_graph:
        del graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result, w


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="the line's headline workload (the other decode workloads are "
                         "reported under configs unless --only)")
    ap.add_argument("--only", action="store_true",
                    help="measure the headline workload alone (no configs, no ceiling sweep)")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--block-size", type=int, default=None,
                    help="tokens per block (default: the workload's own, 16 or 32)")
    ap.add_argument("--layers", type=int, default=None, help="layer cache pools to cycle through")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a graph")
    ap.add_argument("--flush", action="store_true",
                    help="also evict caches before every per-kernel timing launch")
    ap.add_argument("--separate-slot-mapping", action="store_true",
                    help="derive the new tokens' slots and write their K/V in two launches "
                         "(paged_kv_slot_mapping, paged_kv_write) instead of one "
                         "(paged_kv_write_positions)")
    ap.add_argument("--separate-write", action="store_true",
                    help="write the new tokens in a launch of their own (paged_kv_write_positions) "
                         "instead of inside the attention launch")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="forked workloads: read the shared prompt per sequence (the ordinary "
                         "decode) instead of once per group")
    ap.add_argument("--kv-flags", choices=["auto", "streamed", "cached"], default="auto",
                    help="K/V loads: nontemporal streaming or through the caches (auto: cached "
                         "for forked workloads, whose shared blocks are read by several "
                         "workgroups, else streamed)")
    ap.add_argument("--ceilings", metavar="NAME=BYTES,...",
                    help="only measure the streaming-read ceiling at these bytes per launch "
                         "(JSON on stdout); the default run asks a child process for it")
    ap.add_argument("--spread-replays", type=int, default=10,
                    help="extra replays of each timing graph, for p10/p50/p90")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="CPU oracle seconds per setting for the headline workload (a third "
                         "of it for the others)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-plan", action="store_true",
                    help="shared-prefix decode: every attention launch derives its work list "
                         "(no plan launch)")
    ap.add_argument("--no-block-ops", action="store_true",
                    help="skip the copy-on-write and swap copy timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (known bytes), for "
                         "scaling hardware byte counters")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="no GPU: turn rocprofv3 FETCH_SIZE / WRITE_SIZE passes of this workload "
                         "and of --copy-calibration (DIR/{FETCH_SIZE,WRITE_SIZE,cal_FETCH_SIZE,"
                         "cal_WRITE_SIZE}) into HBM bytes per attention launch in "
                         "profiles/attention_traffic.json")
    args = ap.parse_args()

    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.workload)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the decode path runs on a single MI355X.", file=sys.stderr)
        return 2

    import torch

    import workloads

    if args.ceilings:
        if not torch.cuda.is_available():
            log("no GPU visible")
            return 1
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        out = {}
        for item in args.ceilings.split(","):
            name, nbytes = item.split("=")
            out[name] = read_ceiling(dev, int(nbytes))
            log(f"[bench] ceiling {name}: {out[name]['GBps']} GB/s at {nbytes} bytes")
        print(json.dumps(out), flush=True)
        return 0

    # The CPU oracle runs first, before anything initialises the GPU: its
    # all-core setting forks worker processes, which must not inherit a
    # live GPU runtime.
    decode_names = []
    if args.workload not in workloads.PREFILL and not args.copy_calibration:
        decode_names = [args.workload] if args.only else \
            [args.workload] + [n for n in ALL_DECODE if n != args.workload]
    cpu = {}
    if not args.no_cpu_baseline and decode_names:
        cores = cpu_share()
        for name in decode_names:
            w = workloads.make(name, **_block_kw(args))
            secs = args.cpu_seconds if name == args.workload else args.cpu_seconds / 3
            log(f"[bench] CPU oracle on {name}: 1 process, then {cores}")
            one = cpu_baseline(w, secs, 1)
            one["all_cores"] = cpu_baseline(w, secs, cores)
            cpu[name] = one
            del w

    if not args.only and decode_names:
        return all_configs(args, decode_names, cpu)

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.full((1 << 30,), 7, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "launches": 5}))
        return 0

    if args.workload in workloads.PREFILL:
        result = prefill_bench(args, dev)
        if not args.no_cpu_baseline:
            log("[bench] timing the CPU oracle")
            result["cpu_baseline"] = prefill_cpu_baseline(
                workloads.PREFILL[args.workload](**_block_kw(args)), args.cpu_seconds)
        print(json.dumps(result), flush=True)
        return 0

    name = decode_names[0]
    r, _ = decode_bench(name, args, dev, headline=True)
    result = line_of(args, r)
    if name in cpu:
        result["cpu_baseline"] = cpu[name]
    print(json.dumps(result), flush=True)
    return 0


def line_of(args, head: dict) -> dict:
    """The result line's fields for one workload's measurement."""
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "us_per_step": head["us_per_step"],
        "hbm_frac_step": head["hbm_frac_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "accumulate": "f32",
        "data": "synthetic (seeded N(0,1) K/V/q, shuffled block pool)",
        "config": head["config"],
        "roofline": head["roofline"],
        "kernel_us": head["kernel_us"],
        "kernel_us_dist": head["kernel_us_dist"],
        "us_per_step_dist": head["us_per_step_dist"],
        "kernel_source_sha": kernel_source_sha(),
    }
    if "block_ops" in head:
        result["block_ops"] = head["block_ops"]
    return result


def _child(args, extra) -> dict:
    """Run this script in a child process (a fresh GPU context) and parse
    the JSON line it prints; its progress lines go to our stderr."""
    import subprocess
    cmd = [sys.executable, "-u", os.path.abspath(__file__), "--steps", str(args.steps),
           "--warmup", str(args.warmup), "--spread-replays", str(args.spread_replays)]
    for flag in ("flush", "no_graph", "separate_write", "separate_slot_mapping",
                 "no_shared_prefix", "no_plan"):
        if getattr(args, flag):
            cmd.append("--" + flag.replace("_", "-"))
    if args.kv_flags != "auto":
        cmd += ["--kv-flags", args.kv_flags]
    if args.block_size:
        cmd += ["--block-size", str(args.block_size)]
    p = subprocess.run(cmd + extra, stdout=subprocess.PIPE, text=True)
    if p.returncode != 0:
        raise SystemExit(f"[bench] child {' '.join(extra)} failed ({p.returncode})")
    return json.loads(p.stdout.strip().splitlines()[-1])


def all_configs(args, names, cpu) -> int:
    """Every decode workload, each measured by a child process of its own
    (what a process did before carries over: the long-context attention
    measured 4% slower after the other workloads than alone), then the
    streaming-read ceilings at 2 GiB and at each workload's bytes per launch,
    assembled into one line headed by args.workload.  The headline workload
    goes first: the GPU has been idle during the CPU-oracle phase, while
    ~20 s of sustained streaming settles it ~4% slower for the runs after
    (back-to-back processes show the same; 20 s of idle restores it)."""
    runs = {}
    for name in names:
        extra = ["--workload", name, "--only", "--no-cpu-baseline"]
        if name != args.workload or args.no_block_ops:
            extra.append("--no-block-ops")
        runs[name] = _child(args, extra)
    # (each size in a process of its own too: a second 2 GiB sweep in one
    # process measured 5% below the first)
    sizes = {"2GiB": 2 << 30}
    sizes.update({n: r["roofline"]["algorithmic_bytes"] for n, r in runs.items()})
    ceiling = {}
    for k, v in sizes.items():
        ceiling.update(_child(args, ["--ceilings", f"{k}={v}"]))

    result = dict(runs[args.workload])
    result["ceiling"] = {
        "GBps_2GiB": ceiling["2GiB"]["GBps"],
        "frac_of_peak": round(ceiling["2GiB"]["GBps"] / PEAK_HBM_GBPS, 4),
        "kernel": "pkv_read_ceiling (nontemporal 16-byte grid-stride reads; best of grids "
                  "512-3072 x 2 or 4 loads in flight)",
        "size_matched_GBps": ceiling[args.workload]["GBps"],
    }
    result["frac_of_ceiling"] = round(result["roofline"]["achieved"] /
                                      ceiling[args.workload]["GBps"], 4)
    if args.workload in cpu:
        result["cpu_baseline"] = cpu[args.workload]
    configs = {}
    for name, r in runs.items():
        roof = r["roofline"]
        c = {
            "us_per_step": r["us_per_step"],
            "us_per_step_dist": r["us_per_step_dist"],
            "step_GBps": r["value"],
            "kernel_us": r["kernel_us"],
            "kernel_us_dist": {k: v for k, v in r["kernel_us_dist"].items() if k != "what"},
            "attention_GBps": roof["achieved"],
            "attention_logical_GBps": roof["logical_GBps"],
            "roofline": {"frac": roof["frac"], "traffic": roof["traffic"],
                         "kernel": roof["kernel"], "algorithmic_bytes": roof["algorithmic_bytes"],
                         "logical_bytes": roof["logical_bytes"]},
            "ceiling_GBps": ceiling[name]["GBps"],
            "frac_of_ceiling": round(roof["achieved"] / ceiling[name]["GBps"], 4),
            "config": {k: r["config"][k] for k in ("num_seqs", "num_q_heads", "num_kv_heads",
                                                   "head_size", "block_size", "kv_write",
                                                   "attention_path", "kv_flags",
                                                   "layers_cycled")},
            "dtype": r["dtype"],
        }
        if name in cpu:
            c["cpu_baseline"] = cpu[name]
        configs[name] = c
    result["configs"] = configs
    result["measured"] = "each workload and the ceilings in a fresh child process"
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
