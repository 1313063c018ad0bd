"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` takes an object ``o`` exposing the oracle's functions (the
``oracle`` package itself, or a copy with one function replaced by a planted
mistake) and raises ``AssertionError`` when ``o`` disagrees with a fixed fact:
a worked example printed on the pages (``tests/golden``), a closed form, a
library routine, a brute-force evaluation on tiny inputs, or an invariant.
Pins only call ``o``'s primitive functions, so a mistake planted in one of
them is seen by every pin that depends on it.
"""
from __future__ import annotations

import json
import math
import os
from types import SimpleNamespace

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAD = -2**31


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def namespace(module, **replace) -> SimpleNamespace:
    """A copy of the oracle's public functions, some of them replaced."""
    names = [n for n in dir(module) if not n.startswith("_")]
    ns = SimpleNamespace(**{n: getattr(module, n) for n in names})
    for k, v in replace.items():
        setattr(ns, k, v)
    return ns


# ------------------------------------------------------------------ block arithmetic

def pin_block_counts(o) -> None:
    for c in golden("block_counts.json")["cases"]:
        assert o.blocks_needed(c["tokens"], c["block_size"]) == c["blocks"], c
    g = golden("walkthrough_table_50.json")
    assert o.blocks_needed(g["num_tokens"], g["block_size"]) == g["blocks"]
    # one more block exactly when the last one is full
    for B in (1, 4, 16, 32):
        for n in range(0, 5 * B):
            need = o.blocks_needed(n, B)
            assert need * B >= n and (need - 1) * B < max(n, 1)


def pin_waste_bound(o) -> None:
    """Waste is confined to the last block: 0 <= blocks*B - L <= B-1 ([review],
    physical block allocation; [explainer], section 2), and its mean for
    uniform lengths is (B-1)/2, well under 4% of the tokens of long requests."""
    rng = np.random.default_rng(5)
    for B in (4, 16, 32):
        lens = rng.integers(1, 4096, size=2000)
        waste = np.array([o.blocks_needed(int(n), B) * B - int(n) for n in lens])
        assert waste.min() >= 0 and waste.max() <= B - 1
        fills = np.array([o.last_block_fill(int(n), B) for n in lens])
        assert fills.min() >= 1 and fills.max() <= B
        assert np.all(waste == B - fills)
        assert abs(waste.mean() - (B - 1) / 2) < 0.1 * B
    # lengths U[256, 2048] at B=16: mean waste / mean length < 4%
    lens = rng.integers(256, 2049, size=4000)
    waste = sum(o.blocks_needed(int(n), 16) * 16 - int(n) for n in lens)
    assert waste / lens.sum() < 0.04


def pin_worked_example(o) -> None:
    """Prompt of 7 tokens at block size 4 on physical blocks 7 and 1, then two
    decode tokens: the first fills the free slot of block 1, the second opens
    block 3.  Checks where ``slot_of`` + ``write_ref`` put each token's K and V
    against the block/offset the pages give, and the #filled records."""
    g = golden("worked_example_prompt7.json")
    B = g["block_size"]
    table = np.array(g["table_after_second_decode"] + [PAD], dtype=np.int64)
    Hkv, D = 2, 3
    kv = np.full((2, 8, B, Hkv, D), np.nan)
    ntok = len(g["placements"])
    k = np.arange(ntok * Hkv * D, dtype=np.float64).reshape(ntok, Hkv, D) + 1.0
    v = -k
    slots = np.array([o.slot_of(table, p["token"], B) for p in g["placements"]])
    o.write_ref(kv, k, v, slots)
    for i, p in enumerate(g["placements"]):
        assert np.array_equal(kv[0, p["block"], p["offset"]], k[i]), p
        assert np.array_equal(kv[1, p["block"], p["offset"]], v[i]), p
    # nothing else was written
    assert np.isnan(kv).sum() == kv.size - 2 * ntok * Hkv * D
    # the table's #filled records after each step
    for step, n_tok in (("prefill", 7), ("decode1", 8), ("decode2", 9)):
        filled = g["filled"][step]
        assert o.blocks_needed(n_tok, B) == len(filled)
        assert o.last_block_fill(n_tok, B) == filled[-1]
    # the batched form agrees with the per-token form
    sm = o.slot_mapping_ref(table[None, :], np.zeros(ntok, np.int64),
                            np.array([p["token"] for p in g["placements"]]), B)
    assert np.array_equal(sm, slots)
    assert o.slot_of(table, -1, B) == -1
    neg = o.slot_mapping_ref(table[None, :], np.zeros(2, np.int64), np.array([-1, 3]), B)
    assert neg[0] == -1 and neg[1] == slots[3]


def pin_walkthrough_gather(o) -> None:
    """50 tokens at block size 16 on table [10, 21, 45, 67]: reading the
    sequence through the table is the page's ``kv[:, [10,21,45,67], ...]``
    taken in order; the 65th token lands at offset 0 of appended block 89."""
    g = golden("walkthrough_table_50.json")
    B, n = g["block_size"], g["num_tokens"]
    Hkv, D = 2, 4
    NB = 96
    rng = np.random.default_rng(1)
    for layer in range(g["num_layers"]):
        kv = rng.standard_normal((2, NB, B, Hkv, D))
        row = np.full(8, PAD, dtype=np.int64)
        row[:4] = g["table"]
        k, v = o.gather_ref(kv, row, n)
        page_view = kv[:, g["table"], ...].reshape(2, 4 * B, Hkv, D)[:, :n]
        assert np.array_equal(k, page_view[0]) and np.array_equal(v, page_view[1])
    row[4] = g["appended_block"]
    assert o.blocks_needed(n + 15, B) == 5 and o.blocks_needed(n + 14, B) == 4
    slot = o.slot_of(row, 64, B)
    kv = np.zeros((2, NB, B, Hkv, D))
    o.write_ref(kv, np.ones((1, Hkv, D)), 2 * np.ones((1, Hkv, D)), np.array([slot]))
    assert kv[0, g["appended_block"], 0].min() == 1.0 and kv[1, g["appended_block"], 0].min() == 2.0
    assert kv.sum() == 3.0 * Hkv * D


# ------------------------------------------------------------------ sizing

def pin_pool_sizing(o) -> None:
    g = golden("qwen2_pool.json")
    page = o.page_bytes(g["block_size"], g["num_kv_heads"], g["head_size"], g["dtype_bytes"])
    assert page == g["page_size"]
    assert page * g["num_blocks"] == g["tensor_bytes"]
    shape = o.cache_shape_from_bytes(g["tensor_bytes"], g["block_size"], g["num_kv_heads"],
                                     g["head_size"], g["dtype_bytes"])
    assert list(shape) == g["shape"]
    used = g["num_layers"] * g["tensor_bytes"]
    assert used <= g["gpu_bytes"] * g["utilization"]
    # the block count that memory for exactly this pool (plus any slack below
    # one block of every layer) yields
    for slack in (0, page * g["num_layers"] - 1):
        assert o.num_blocks_for(used + slack, page, g["num_layers"]) == g["num_blocks"]


def pin_opt13b_bytes(o) -> None:
    g = golden("opt13b_kv.json")
    m = g["model_shape_not_on_pages"]
    per_tok = o.kv_bytes_per_token(m["num_layers"], m["num_heads"], m["head_size"], m["dtype_bytes"])
    assert per_tok == g["kv_per_token_kb_approx"] * 1024
    per_seq = per_tok * g["sequence_tokens"]
    assert abs(per_seq / 2**30 - g["kv_per_sequence_gb_approx"]) < 0.05 * g["kv_per_sequence_gb_approx"]
    lo, hi = g["requests_range"]
    assert lo <= g["gpu_gb"] * 1e9 / per_seq <= hi
    # per layer, the page formula gives the same bytes per token
    assert o.page_bytes(1, m["num_heads"], m["head_size"], m["dtype_bytes"]) * m["num_layers"] == per_tok


# ------------------------------------------------------------------ element widening

def pin_bf16_widening(o) -> None:
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x3F81: 1.0078125, 0x4049: 3.140625,
             0x0001: 2.0 ** -133, 0x8000: -0.0, 0x7F7F: 3.3895313892515355e38}
    bits = np.array(list(cases), dtype=np.uint16)
    got = o.to_f64(bits, "bf16")
    assert np.array_equal(got, np.array(list(cases.values())))
    assert np.isinf(o.to_f64(np.array([0x7F80], np.uint16), "bf16"))[0]
    x = np.array([0.1, -3.5, 1e-30], dtype=np.float32)
    assert np.array_equal(o.to_f64(x, "f32"), x.astype(np.float64))


# ------------------------------------------------------------------ attention

def _brute_attention(q, K, V, scale, kv_head):
    """Scalar loops over contiguous K/V (tiny inputs only)."""
    Hq, D = len(q), len(q[0])
    L = len(K)
    out = [[0.0] * D for _ in range(Hq)]
    for h in range(Hq):
        g = kv_head[h]
        z = []
        for t in range(L):
            acc = 0.0
            for d in range(D):
                acc += q[h][d] * K[t][g][d]
            z.append(scale * acc)
        top = max(z)
        e = [math.exp(x - top) for x in z]
        tot = sum(e)
        for d in range(D):
            out[h][d] = sum(e[t] * V[t][g][d] for t in range(L)) / tot
    return np.array(out)


def pin_attention_bruteforce(o) -> None:
    rng = np.random.default_rng(7)
    for (Hq, Hkv, D, L) in ((1, 1, 4, 1), (2, 2, 8, 5), (4, 2, 8, 17), (6, 3, 16, 40), (8, 1, 5, 9)):
        q = rng.standard_normal((Hq, D))
        K = rng.standard_normal((L, Hkv, D))
        V = rng.standard_normal((L, Hkv, D))
        scale = 0.37
        G = Hq // Hkv
        ref = _brute_attention(q.tolist(), K.tolist(), V.tolist(), scale, [h // G for h in range(Hq)])
        got = o.attention_ref(q, K, V, scale)
        assert np.abs(got - ref).max() < 1e-12, (Hq, Hkv, D, L)


def pin_attention_sdpa(o) -> None:
    """Against torch's scaled_dot_product_attention on the CPU in float64, with
    each kv head repeated for its group of query heads."""
    import torch
    rng = np.random.default_rng(11)
    for (Hq, Hkv, D, L) in ((4, 4, 64, 33), (14, 2, 64, 100), (32, 8, 128, 70), (8, 2, 16, 1)):
        q = rng.standard_normal((Hq, D))
        K = rng.standard_normal((L, Hkv, D)) * 2.0
        V = rng.standard_normal((L, Hkv, D))
        scale = 1.0 / math.sqrt(D)
        G = Hq // Hkv
        tq = torch.from_numpy(q)[None, :, None, :]
        tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)[0, :, 0, :].numpy()
        got = o.attention_ref(q, K, V, scale)
        assert np.abs(got - ref).max() < 1e-12, (Hq, Hkv, D, L)


def pin_attention_closed_forms(o) -> None:
    rng = np.random.default_rng(13)
    Hq, Hkv, D = 8, 2, 16
    # one token: the output is that token's value, exactly
    q = rng.standard_normal((Hq, D))
    K = rng.standard_normal((1, Hkv, D))
    V = rng.standard_normal((1, Hkv, D))
    got = o.attention_ref(q, K, V, 0.5)
    assert np.array_equal(got, np.repeat(V[0], Hq // Hkv, axis=0))
    # zero query, or all keys equal: the mean of the values
    L = 23
    K = rng.standard_normal((L, Hkv, D))
    V = rng.standard_normal((L, Hkv, D))
    got = o.attention_ref(np.zeros((Hq, D)), K, V, 0.5)
    assert np.abs(got - np.repeat(V.mean(axis=0), Hq // Hkv, axis=0)).max() < 1e-14
    Keq = np.repeat(K[:1], L, axis=0)
    got = o.attention_ref(q, Keq, V, 0.5)
    assert np.abs(got - np.repeat(V.mean(axis=0), Hq // Hkv, axis=0)).max() < 1e-14
    # one key aligned with the query far above the rest: its value, to e^-50
    K = rng.standard_normal((L, 1, D)) * 1e-3
    qv = rng.standard_normal(D)
    qv /= np.linalg.norm(qv)
    K[9, 0] = 50.0 * qv
    got = o.attention_ref(qv[None, :], K, V[:, :1], 1.0)
    assert np.abs(got[0] - V[9, 0]).max() < L * math.exp(-49.0)
    # no tokens: zeros
    assert not o.attention_ref(q, np.zeros((0, Hkv, D)), np.zeros((0, Hkv, D)), 0.5).any()
    # the scale multiplies the scores: scale s with q equals scale 1 with s*q
    K = rng.standard_normal((L, Hkv, D))
    a = o.attention_ref(q, K, V, 0.3)
    b = o.attention_ref(0.3 * q, K, V, 1.0)
    assert np.abs(a - b).max() < 1e-13


def _toy_paged(rng, lens, B, Hkv, D, NB, share=None):
    """Place contiguous K/V of each sequence into a random pool (test helper;
    computes placements by a position loop independent of the oracle)."""
    S = len(lens)
    width = max(1, max((n + B - 1) // B for n in lens))
    tables = np.full((S, width), PAD, dtype=np.int64)
    kv = np.full((2, NB, B, Hkv, D), np.nan)
    perm = list(rng.permutation(NB))
    Ks, Vs = [], []
    for s, n in enumerate(lens):
        K = rng.standard_normal((n, Hkv, D))
        V = rng.standard_normal((n, Hkv, D))
        Ks.append(K)
        Vs.append(V)
        j = -1
        for t in range(n):
            if t % B == 0:
                j += 1
                tables[s, j] = perm.pop()
            kv[0, tables[s, j], t % B] = K[t]
            kv[1, tables[s, j], t % B] = V[t]
    return kv, tables, Ks, Vs


def pin_paged_invariants(o) -> None:
    """Reading through the table gives the contiguous sequence; relabelling
    physical blocks or aliasing a shared prefix changes nothing; NaN in unused
    slots and padded table entries are never read."""
    rng = np.random.default_rng(17)
    B, Hkv, D, Hq = 16, 2, 8, 6
    lens = [1, 15, 16, 17, 60, 129]
    NB = 40
    kv, tables, Ks, Vs = _toy_paged(rng, lens, B, Hkv, D, NB)
    q = rng.standard_normal((len(lens), Hq, D))
    outs = []
    for s, n in enumerate(lens):
        k, v = o.gather_ref(kv, tables[s], n)
        assert np.array_equal(k, Ks[s]) and np.array_equal(v, Vs[s])
        outs.append(o.attention_ref(q[s], k, v, 0.25))
    # relabel the pool: block b moves to perm[b]
    perm = rng.permutation(NB)
    kv2 = np.empty_like(kv)
    kv2[:, perm] = kv
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], PAD)
    for s, n in enumerate(lens):
        k, v = o.gather_ref(kv2, t2[s], n)
        assert np.array_equal(o.attention_ref(q[s], k, v, 0.25), outs[s])
    # aliasing: three forks share the first two blocks of a 40-token prompt
    prompt = 32
    base_k = rng.standard_normal((prompt, Hkv, D))
    base_v = rng.standard_normal((prompt, Hkv, D))
    kv3 = np.full((2, 16, B, Hkv, D), np.nan)
    kv3[0, 3], kv3[0, 5] = base_k[:16], base_k[16:]
    kv3[1, 3], kv3[1, 5] = base_v[:16], base_v[16:]
    for f, (blk, extra) in enumerate(((7, 4), (9, 0), (11, 13))):
        ek = rng.standard_normal((extra, Hkv, D))
        ev = rng.standard_normal((extra, Hkv, D))
        kv3[0, blk, :extra], kv3[1, blk, :extra] = ek, ev
        row = np.array([3, 5, blk if extra else PAD, PAD], dtype=np.int64)
        k, v = o.gather_ref(kv3, row, prompt + extra)
        private_k = np.concatenate([base_k, ek])
        private_v = np.concatenate([base_v, ev])
        assert np.array_equal(o.attention_ref(q[0], k, v, 0.25),
                              o.attention_ref(q[0], private_k, private_v, 0.25))


def pin_split_merge(o) -> None:
    rng = np.random.default_rng(19)
    for (Hq, Hkv, D, L, B) in ((8, 2, 16, 1000, 16), (4, 4, 8, 77, 16), (16, 2, 32, 1500, 32)):
        q = rng.standard_normal((Hq, D))
        K = rng.standard_normal((L, Hkv, D)) * 1.5
        V = rng.standard_normal((L, Hkv, D))
        full = o.attention_ref(q, K, V, 0.2)
        for P in (B, 64, 512, L, L + 5):
            stats = o.partition_stats_ref(q, K, V, 0.2, P)
            assert len(stats) == o.blocks_needed(L, P)
            merged = o.merge_ref(stats)
            assert np.abs(merged - full).max() < 1e-12, (L, P)
        # partition outputs are themselves attention over their slices
        stats = o.partition_stats_ref(q, K, V, 0.2, 64)
        m0, l0, o0 = stats[1]
        assert np.abs(o0 - o.attention_ref(q, K[64:128], V[64:128], 0.2)).max() < 1e-12
        G = Hq // Hkv
        z = np.stack([0.2 * (K[64:128, h // G, :] @ q[h]) for h in range(Hq)])
        assert np.abs(m0 - z.max(axis=1)).max() < 1e-14
        assert np.abs(l0 - np.exp(z - z.max(axis=1, keepdims=True)).sum(axis=1)).max() < 1e-12


# ------------------------------------------------------------------ block manager

def _free_order(n, head):
    return list(head) + [b for b in range(n) if b not in head]


def _cached_blocks(m):
    return sorted(m.cache.values())


def pin_cow_parallel_samples(o) -> None:
    """Two samples of one prompt share its blocks; the first writer of a
    shared block copies it, the last one writes in place ([review] worked
    example, tests/golden/cow_parallel_samples.json)."""
    g = golden("cow_parallel_samples.json")
    m = o.RefBlockManager(g["num_blocks"], g["block_size"],
                          free_order=_free_order(g["num_blocks"], g["free_order_head"]))
    m.allocate(1, g["prompt"])
    m.fork(1, 2)
    e = g["after_prefill_and_fork"]
    assert m.table(1) == e["table"] and m.table(2) == e["table"]
    assert all(m.ref[int(b)] == r for b, r in e["ref"].items())
    for sid, key in ((1, "A1_writes"), (2, "A2_writes")):
        e = g[key]
        slots, copies = m.append(sid, [e["token"]])
        assert slots == [e["slot"]], (key, slots)
        assert [list(c) for c in copies] == e["copies"], (key, copies)
        assert m.table(sid) == e["table"]
        assert all(m.ref[int(b)] == r for b, r in e["ref"].items())


def pin_prefix_cache_timeline(o) -> None:
    """Times 1-6 of [walkthrough]'s prefix-cache timeline: hits, the free
    queue order after reverse-order frees, eviction of reused cached blocks
    (tests/golden/prefix_cache_timeline.json)."""
    g = golden("prefix_cache_timeline.json")
    m = o.RefBlockManager(g["num_blocks"], g["block_size"])
    for st in g["steps"]:
        if st["op"] == "allocate":
            assert m.allocate(st["seq"], st["tokens"]) == st["cached_tokens"], st["time"]
        elif st["op"] == "append":
            m.append(st["seq"], st["tokens"])
        else:
            m.free_seq(st["seq"])
        if "table" in st:
            assert m.table(st["seq"]) == st["table"], (st["time"], m.table(st["seq"]))
        if "free_queue" in st:
            assert m.free == st["free_queue"], (st["time"], m.free)
        if "cached_blocks" in st:
            assert _cached_blocks(m) == st["cached_blocks"], (st["time"], _cached_blocks(m))
        if "still_cached" in st:
            assert set(st["still_cached"]) <= set(_cached_blocks(m)), st["time"]
    # time 6 reused block 3, so its old content is no longer a hit
    assert 3 not in [m.cache.get(h) for h in m.cache if m.cache[h] == 3 and m.hash_of[3] is not None] or \
        m.hash_of[3] is None


def pin_prefix_hit_table_50(o) -> None:
    """[walkthrough] 'ブロック割当のロジック': 50 tokens at B = 16 get table
    [10, 21, 45, 67] with the first two blocks from the prefix cache; token 64
    takes block 89 (tests/golden/prefix_hit_table_50.json)."""
    g = golden("prefix_hit_table_50.json")
    m = o.RefBlockManager(g["num_blocks"], g["block_size"],
                          free_order=_free_order(g["num_blocks"], g["free_order_head"]))
    m.allocate(7, g["earlier_request"])
    m.free_seq(7)
    assert m.allocate(8, g["request"]) == g["cached_tokens"]
    assert m.table(8) == g["table"]
    slots, copies = m.append(8, g["decode_tokens"])
    assert m.table(8) == g["table_after_decode"] and not copies
    first = g["first_token_in_89"]
    assert slots[first - len(g["request"])] == 89 * g["block_size"]
    # the same 32 tokens again: hits are looked up over num_tokens - 1 tokens
    # (find_longest_cache_hit's max_length), so the last block is computed
    assert m.allocate(9, g["earlier_request"]) == g["block_size"]


def pin_block_hash_chain(o) -> None:
    """A block's hash depends on every earlier token and on nothing else:
    equal prefixes hash equally, any earlier change changes every later hash."""
    rng = np.random.default_rng(5)
    toks = rng.integers(0, 1000, 64).tolist()

    def chain(t):
        out, h = [], o.NONE_HASH
        for i in range(len(t) // 16):
            h = o.block_hash(h, t[16 * i:16 * (i + 1)])
            out.append(h)
        return out

    base = chain(toks)
    assert len(set(base)) == 4 and all(len(h) == 32 for h in base)
    assert chain(list(toks)) == base
    for pos in (0, 17, 63):
        t2 = list(toks)
        t2[pos] += 1
        c2 = chain(t2)
        b = pos // 16
        assert c2[:b] == base[:b] and all(x != y for x, y in zip(c2[b:], base[b:]))
    # the same 16 tokens under another parent hash differently
    assert o.block_hash(o.NONE_HASH, toks[16:32]) != base[1]


def _simulate(o, seed, N=24, B=4, ncpu=24, steps=300):
    """Random allocate / append / fork / free / swap sequences on a small pool,
    with the pool's contents modelled as token ids per slot (copy-on-write and
    swap copies applied as the manager asks).  After every operation: reading
    each sequence through its table gives its own tokens; reference counts
    equal the table entries pointing at each block; the free queue is exactly
    the unreferenced blocks; a refused operation changed nothing."""
    rng = np.random.default_rng(seed)
    m = o.RefBlockManager(N, B, num_cpu_blocks=ncpu)
    gpu = np.full(N * B, -1, dtype=np.int64)
    cpu = np.full(ncpu * B, -1, dtype=np.int64)
    toks = {}
    nxt = 0
    vocab = [list(rng.integers(0, 50, 40)) for _ in range(3)]  # shared prompt stems

    def check():
        for sid, t in toks.items():
            s = m.seqs[sid]
            pool = cpu if s.swapped else gpu
            got = [int(pool[s.table[p // B] * B + p % B]) for p in range(len(t))]
            assert got == t, (sid, got, t)
            assert len(s.table) == -(-len(t) // B)
        refs = [0] * N
        for s in m.seqs.values():
            if not s.swapped:
                for b in s.table:
                    refs[b] += 1
        assert refs == m.ref, (refs, m.ref)
        assert sorted(m.free) == [b for b in range(N) if refs[b] == 0]
        for h, b in m.cache.items():
            assert m.hash_of[b] == h

    def state():
        return (list(m.ref), list(m.hash_of), dict(m.cache), list(m.free), list(m.cpu_free),
                list(m.cpu_ref), {i: (list(s.table), list(s.tokens), list(s.hashes), s.swapped)
                                  for i, s in m.seqs.items()})

    for _ in range(steps):
        snap = state()
        op = rng.integers(0, 6)
        live = [i for i in toks if not m.seqs[i].swapped]
        try:
            if op == 0 or not toks:
                stem = vocab[rng.integers(0, 3)]
                n = int(rng.integers(1, 20))
                t = [int(x) for x in stem[:rng.integers(0, n + 1)]]
                t += [int(x) for x in rng.integers(100, 200, n - len(t))]
                sid = nxt
                nxt += 1
                cached = m.allocate(sid, t)
                # whole cached blocks, and the last token is always computed
                assert cached % B == 0 and (cached < len(t) or not t)
                for p in range(cached, len(t)):
                    gpu[m.table(sid)[p // B] * B + p % B] = t[p]
                toks[sid] = t
            elif op == 1 and live:
                sid = live[rng.integers(0, len(live))]
                new = [int(x) for x in rng.integers(100, 200, rng.integers(1, 6))]
                slots, copies = m.append(sid, new)
                for s_, d_ in copies:
                    gpu[d_ * B:(d_ + 1) * B] = gpu[s_ * B:(s_ + 1) * B]
                for sl, tk in zip(slots, new):
                    assert m.ref[sl // B] == 1  # nobody else sees the written block
                    gpu[sl] = tk
                toks[sid] = toks[sid] + new
            elif op == 2 and live:
                sid = live[rng.integers(0, len(live))]
                m.fork(sid, nxt)
                toks[nxt] = list(toks[sid])
                nxt += 1
            elif op == 3:
                sid = list(toks)[rng.integers(0, len(toks))]
                m.free_seq(sid)
                del toks[sid]
            elif op == 4 and live:
                # a sequence and everything sharing blocks with it
                sid = live[rng.integers(0, len(live))]
                group = {sid}
                grew = True
                while grew:
                    blocks = {b for i in group for b in m.seqs[i].table}
                    more = {i for i in live if set(m.seqs[i].table) & blocks}
                    grew = not more <= group
                    group |= more
                for g_, c_ in m.swap_out(sorted(group)):
                    cpu[c_ * B:(c_ + 1) * B] = gpu[g_ * B:(g_ + 1) * B]
            elif op == 5:
                swapped = [i for i in toks if m.seqs[i].swapped]
                if swapped:
                    group, grew = {swapped[0]}, True
                    while grew:
                        blocks = {b for i in group for b in m.seqs[i].table}
                        more = {i for i in swapped if set(m.seqs[i].table) & blocks}
                        grew = not more <= group
                        group |= more
                    group = sorted(group)
                    for c_, g_ in m.swap_in(group):
                        gpu[g_ * B:(g_ + 1) * B] = cpu[c_ * B:(c_ + 1) * B]
        except o.OutOfBlocks:
            assert state() == snap, "a refused operation changed the state"
        check()


def pin_block_manager_invariants(o) -> None:
    for seed in range(4):
        _simulate(o, seed)


def pin_copy_blocks(o) -> None:
    """Block copies move whole blocks (keys and values) and nothing else."""
    rng = np.random.default_rng(9)
    kv = rng.standard_normal((2, 6, 4, 2, 3))
    before = kv.copy()
    o.copy_blocks_ref(kv, [(1, 4), (5, 0)])
    assert np.array_equal(kv[:, 4], before[:, 1]) and np.array_equal(kv[:, 0], before[:, 5])
    assert np.array_equal(kv[:, [1, 2, 3, 5]], before[:, [1, 2, 3, 5]])
    host = np.zeros((2, 3, 4, 2, 3))
    o.copy_blocks_ref(before, [(2, 1)], dst=host)
    assert np.array_equal(host[:, 1], before[:, 2]) and not host[:, [0, 2]].any()


# ------------------------------------------------------------------ prefill

def _concat_queries(rng, chunk_lens, Hq, D):
    starts = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int64)
    return _f32(rng.standard_normal((int(starts[-1]), Hq, D))), starts


def _f32(x):
    """float64 values that float32 holds exactly (so "f32" inputs widen back
    to the same numbers)."""
    return np.asarray(x).astype(np.float32).astype(np.float64)


def _toy_paged_f32(rng, lens, B, Hkv, D, NB):
    kv, tables, Ks, Vs = _toy_paged(rng, lens, B, Hkv, D, NB)
    return _f32(kv), tables, [_f32(k) for k in Ks], [_f32(v) for v in Vs]


def pin_prefill_sdpa(o) -> None:
    """Whole prompts (each chunk is its entire sequence), several joined in one
    batch, against torch's causal scaled_dot_product_attention on the CPU in
    float64, one sequence at a time from its contiguous K/V."""
    import torch
    rng = np.random.default_rng(31)
    for (Hq, Hkv, D, B, lens) in ((4, 4, 16, 4, [5, 17, 1]), (6, 2, 8, 16, [40, 16]),
                                  (8, 1, 32, 8, [33])):
        NB = sum((n + B - 1) // B for n in lens) + 3
        kv, tables, Ks, Vs = _toy_paged_f32(rng, lens, B, Hkv, D, NB)
        q, starts = _concat_queries(rng, lens, Hq, D)
        scale = 1.0 / math.sqrt(D)
        got = o.prefill_attention_ref(q, kv, tables, np.array(lens), starts, scale, "f32")
        G = Hq // Hkv
        for s, n in enumerate(lens):
            tq = torch.from_numpy(q[starts[s]:starts[s + 1]]).permute(1, 0, 2)[None]
            tk = torch.from_numpy(Ks[s]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
            tv = torch.from_numpy(Vs[s]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, is_causal=True, scale=scale)[0].permute(1, 0, 2).numpy()
            assert np.abs(got[starts[s]:starts[s + 1]] - ref).max() < 1e-12, (Hq, Hkv, D, n)


def pin_prefill_chunks(o) -> None:
    """A chunk that continues a sequence gives the rows a whole-prompt pass
    gives for the same positions (chunked prefill), and a chunk of one token
    is the decode step."""
    rng = np.random.default_rng(37)
    Hq, Hkv, D, B = 6, 3, 8, 4
    lens = [9, 30, 1, 16]
    kv, tables, _, _ = _toy_paged_f32(rng, lens, B, Hkv, D, 40)
    L = np.array(lens)
    q_all, starts_all = _concat_queries(rng, lens, Hq, D)
    whole = o.prefill_attention_ref(q_all, kv, tables, L, starts_all, 0.4, "f32")
    for chunk in ([4, 11, 1, 16], [1, 30, 1, 3], [9, 1, 1, 1]):
        starts = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int64)
        rows = np.concatenate([np.arange(starts_all[s + 1] - c, starts_all[s + 1])
                               for s, c in enumerate(chunk)])
        got = o.prefill_attention_ref(q_all[rows], kv, tables, L, starts, 0.4, "f32")
        assert np.abs(got - whole[rows]).max() < 1e-13, chunk
    last = starts_all[1:] - 1
    dec = o.paged_attention_ref(q_all[last], kv, tables, L, 0.4, "f32")
    got = o.prefill_attention_ref(q_all[last], kv, tables, L, np.arange(len(lens) + 1), 0.4, "f32")
    assert np.abs(got - dec).max() < 1e-13


def pin_prefill_closed_forms(o) -> None:
    """The first token of a prompt sees only itself (its value, exactly); with
    every key equal, the token at position p gets the mean of values 0..p."""
    rng = np.random.default_rng(41)
    Hq, Hkv, D, B, n = 4, 2, 8, 4, 13
    kv, tables, Ks, Vs = _toy_paged_f32(rng, [n], B, Hkv, D, 8)
    q, starts = _concat_queries(rng, [n], Hq, D)
    got = o.prefill_attention_ref(q, kv, tables, np.array([n]), starts, 0.5, "f32")
    assert np.array_equal(got[0], np.repeat(Vs[0][0], Hq // Hkv, axis=0))
    for t in range(n):  # all keys equal
        b = tables[0, t // B]
        kv[0, b, t % B] = Ks[0][0]
    got = o.prefill_attention_ref(q, kv, tables, np.array([n]), starts, 0.5, "f32")
    for p in range(n):
        mean = np.repeat(Vs[0][:p + 1].mean(axis=0), Hq // Hkv, axis=0)
        assert np.abs(got[p] - mean).max() < 1e-14, p
    assert list(o.chunk_positions(10, 3)) == [7, 8, 9] and len(o.chunk_positions(4, 0)) == 0


ALL_PINS = [
    pin_block_counts,
    pin_waste_bound,
    pin_worked_example,
    pin_walkthrough_gather,
    pin_pool_sizing,
    pin_opt13b_bytes,
    pin_bf16_widening,
    pin_attention_bruteforce,
    pin_attention_sdpa,
    pin_attention_closed_forms,
    pin_paged_invariants,
    pin_split_merge,
    pin_cow_parallel_samples,
    pin_prefix_cache_timeline,
    pin_prefix_hit_table_50,
    pin_block_hash_chain,
    pin_block_manager_invariants,
    pin_copy_blocks,
    pin_prefill_sdpa,
    pin_prefill_chunks,
    pin_prefill_closed_forms,
]
