"""The library's host block manager (C++, through the C ABI) against the
oracle's: identical tables, slots, copy lists, reference counts, free-queue
order, block hashes and cached blocks after every operation of random
sessions, and the pages' worked examples checked directly.  Host code only:
runs without a GPU."""
import numpy as np
import pytest

import oracle
from paged_kv_cache_81_amd.block_manager import BlockManager, NoFreeBlocks
from tests.oracle_pins import golden


def _free_order(n, head):
    return list(head) + [b for b in range(n) if b not in head]


def _same_state(lib, ref, live):
    assert lib.ref_counts() == ref.ref
    assert lib.free_queue() == ref.free
    assert lib.cached_blocks() == sorted(ref.cache.values())
    for b in range(ref.N):
        assert lib.block_hash(b) == ref.hash_of[b], b
    for sid in live:
        assert lib.table(sid) == ref.table(sid), sid
        assert lib.num_tokens(sid) == ref.num_tokens(sid)
        assert lib.is_swapped(sid) == ref.seqs[sid].swapped


def test_cow_parallel_samples_example():
    g = golden("cow_parallel_samples.json")
    m = BlockManager(g["num_blocks"], g["block_size"],
                     free_order=_free_order(g["num_blocks"], g["free_order_head"]))
    m.allocate(1, g["prompt"])
    m.fork(1, 2)
    assert m.table(1) == m.table(2) == g["after_prefill_and_fork"]["table"]
    for sid, key in ((1, "A1_writes"), (2, "A2_writes")):
        e = g[key]
        slots, copies = m.append(sid, [e["token"]])
        assert slots == [e["slot"]] and [list(c) for c in copies] == e["copies"]
        assert m.table(sid) == e["table"]
        assert all(m.ref_count(int(b)) == r for b, r in e["ref"].items())


def test_prefix_cache_timeline_example():
    g = golden("prefix_cache_timeline.json")
    m = BlockManager(g["num_blocks"], g["block_size"])
    for st in g["steps"]:
        if st["op"] == "allocate":
            assert m.allocate(st["seq"], st["tokens"]) == st["cached_tokens"]
        elif st["op"] == "append":
            m.append(st["seq"], st["tokens"])
        else:
            m.free(st["seq"])
        if "table" in st:
            assert m.table(st["seq"]) == st["table"], st["time"]
        if "free_queue" in st:
            assert m.free_queue() == st["free_queue"], st["time"]
        if "cached_blocks" in st:
            assert m.cached_blocks() == st["cached_blocks"], st["time"]


def test_prefix_hit_table_50_example():
    g = golden("prefix_hit_table_50.json")
    m = BlockManager(g["num_blocks"], g["block_size"],
                     free_order=_free_order(g["num_blocks"], g["free_order_head"]))
    m.allocate(7, g["earlier_request"])
    m.free(7)
    assert m.allocate(8, g["request"]) == g["cached_tokens"]
    assert m.table(8) == g["table"]
    slots, copies = m.append(8, g["decode_tokens"])
    assert m.table(8) == g["table_after_decode"] and not copies
    assert slots[g["first_token_in_89"] - len(g["request"])] == 89 * g["block_size"]


def test_block_hash_is_sha256_chain():
    """The native SHA-256 chain hash equals the oracle's (hashlib) bit for bit."""
    m = BlockManager(16, 4)
    toks = list(range(1000, 1013))
    m.allocate(0, toks)
    h = oracle.NONE_HASH
    for i, b in enumerate(m.table(0)[:3]):
        h = oracle.block_hash(h, toks[4 * i:4 * i + 4])
        assert m.block_hash(b) == h
    assert m.block_hash(m.table(0)[3]) is None  # partial block


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("prefix", [True, False])
def test_random_sessions_match_oracle(seed, prefix):
    rng = np.random.default_rng(100 + seed)
    N, B, ncpu = 40, 4, 32
    lib = BlockManager(N, B, prefix_caching=prefix, num_cpu_blocks=ncpu)
    ref = oracle.RefBlockManager(N, B, prefix_caching=prefix, num_cpu_blocks=ncpu)
    stems = [rng.integers(0, 50, 40).tolist() for _ in range(3)]
    live, nxt = [], 0
    for step in range(400):
        op = int(rng.integers(0, 6))
        resident = [i for i in live if not ref.seqs[i].swapped]
        try:
            if op == 0 or not live:
                n = int(rng.integers(1, 24))
                t = stems[rng.integers(0, 3)][:rng.integers(0, n + 1)]
                t = t + rng.integers(100, 200, n - len(t)).tolist()
                try:
                    want = ref.allocate(nxt, t)
                except oracle.OutOfBlocks:
                    with pytest.raises(NoFreeBlocks):
                        lib.allocate(nxt, t)
                    continue
                assert lib.allocate(nxt, t) == want
                live.append(nxt)
                nxt += 1
            elif op == 1 and resident:
                sid = resident[rng.integers(0, len(resident))]
                new = rng.integers(100, 200, rng.integers(1, 7)).tolist()
                try:
                    want = ref.append(sid, new)
                except oracle.OutOfBlocks:
                    with pytest.raises(NoFreeBlocks):
                        lib.append(sid, new)
                    continue
                got = lib.append(sid, new)
                assert got[0] == want[0] and got[1] == [tuple(c) for c in want[1]]
            elif op == 2 and resident:
                sid = resident[rng.integers(0, len(resident))]
                ref.fork(sid, nxt)
                lib.fork(sid, nxt)
                live.append(nxt)
                nxt += 1
            elif op == 3 and live:
                sid = live.pop(int(rng.integers(0, len(live))))
                ref.free_seq(sid)
                lib.free(sid)
            elif op == 4 and resident:
                sid = resident[rng.integers(0, len(resident))]
                group, grew = {sid}, True
                while grew:
                    blocks = {b for i in group for b in ref.seqs[i].table}
                    more = {i for i in resident if set(ref.seqs[i].table) & blocks}
                    grew = not more <= group
                    group |= more
                group = sorted(group)
                try:
                    want = ref.swap_out(group)
                except oracle.OutOfBlocks:
                    with pytest.raises(NoFreeBlocks):
                        lib.swap_out(group)
                    continue
                assert lib.swap_out(group) == [tuple(c) for c in want]
            elif op == 5:
                swapped = [i for i in live if ref.seqs[i].swapped]
                if swapped:
                    group, grew = {swapped[0]}, True
                    while grew:
                        blocks = {b for i in group for b in ref.seqs[i].table}
                        more = {i for i in swapped if set(ref.seqs[i].table) & blocks}
                        grew = not more <= group
                        group |= more
                    group = sorted(group)
                    try:
                        want = ref.swap_in(group)
                    except oracle.OutOfBlocks:
                        with pytest.raises(NoFreeBlocks):
                            lib.swap_in(group)
                        continue
                    assert lib.swap_in(group) == [tuple(c) for c in want]
        finally:
            _same_state(lib, ref, live)
        for sid in [i for i in live if not ref.seqs[i].swapped][:3]:
            n = ref.num_tokens(sid)
            assert lib.slots(sid, 0, n) == ref.slots(sid, 0, n)


def test_batch_tables_and_errors():
    m = BlockManager(32, 16)
    m.allocate(3, list(range(40)))
    m.allocate(5, list(range(1000, 1017)))
    tables, lens = m.batch_tables([5, 3], 4)
    assert lens.tolist() == [17, 40]
    assert tables[1, :3].tolist() == m.table(3) and tables[1, 3] == -2**31
    assert tables[0, :2].tolist() == m.table(5) and (tables[0, 2:] == -2**31).all()
    from paged_kv_cache_81_amd._lib import PagedKVError
    with pytest.raises(PagedKVError):
        m.allocate(3, [1])          # sequence exists
    with pytest.raises(PagedKVError):
        m.append(99, [1])           # no such sequence
    with pytest.raises(PagedKVError):
        m.batch_tables([3], 2)      # wider than the table
    with pytest.raises(PagedKVError):
        BlockManager(4, 4, free_order=[0, 1, 1, 2])
    before = (m.free_queue(), m.ref_counts(), m.table(3))
    with pytest.raises(NoFreeBlocks):
        m.allocate(7, list(range(30 * 16)))
    assert (m.free_queue(), m.ref_counts(), m.table(3)) == before
