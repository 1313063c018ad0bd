"""Plant plausible mistakes in copies of the oracle's functions (on the CPU)
and check that at least one pin fails for each: the pins are sharp enough to
catch a dropped term, a wrong sign or index, or a transposed operand."""
import numpy as np
import pytest

import oracle
from oracle import paged_attention as pa
from tests import oracle_pins as pins


def _floor_blocks(n, b):
    return n // b


def _slot_swapped(row, pos, B):
    if pos < 0:
        return -1
    lb, off = divmod(int(pos), B)
    return int(row[off % len(row)]) * B + lb


def _slot_off_by_one(row, pos, B):
    if pos < 0:
        return -1
    lb, off = divmod(int(pos), B)
    return int(row[lb]) * B + off + 1


def _write_kv_swapped(kv, k, v, slot_mapping):
    pa.write_ref(kv, v, k, slot_mapping)


def _gather_wrong_index(kv, row, L):
    B = kv.shape[2]
    pos = np.arange(L)
    phys = np.asarray(row)[pos % B % max(1, (L + B - 1) // B)]
    return kv[0, phys, pos % B], kv[1, phys, pos % B]


def _attn_no_scale(q, K, V, scale):
    return pa.attention_ref(q, K, V, 1.0)


def _attn_wrong_head_map(q, K, V, scale):
    Hq, D = q.shape
    Hkv = K.shape[1]
    out = np.zeros((Hq, D))
    if K.shape[0] == 0:
        return out
    for h in range(Hq):
        g = h % Hkv
        z = scale * (K[:, g, :] @ q[h])
        w = np.exp(z - z.max())
        out[h] = (w / w.sum()) @ V[:, g, :]
    return out


def _attn_sign(q, K, V, scale):
    return pa.attention_ref(-q, K, V, scale)


def _attn_kv_transposed(q, K, V, scale):
    return pa.attention_ref(q, V, K, scale)


def _attn_unnormalised(q, K, V, scale):
    Hq, D = q.shape
    out = np.zeros((Hq, D))
    G = Hq // K.shape[1]
    if K.shape[0] == 0:
        return out
    for h in range(Hq):
        z = scale * (K[:, h // G, :] @ q[h])
        out[h] = np.exp(z - z.max()) @ V[:, h // G, :]
    return out


def _merge_no_exp(stats):
    ls = np.stack([l for _, l, _ in stats])
    os_ = np.stack([o for _, _, o in stats])
    return (ls[:, :, None] * os_).sum(0) / ls.sum(0)[:, None]


def _merge_no_l(stats):
    ms = np.stack([m for m, _, _ in stats])
    os_ = np.stack([o for _, _, o in stats])
    w = np.exp(ms - ms.max(0))
    return (w[:, :, None] * os_).sum(0) / w.sum(0)[:, None]


def _page_no_kv_factor(B, H, D, nbytes):
    return B * H * D * nbytes


def _widen_wrong_shift(x, dtype):
    if dtype == "bf16":
        return (np.asarray(x, np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return pa.to_f64(x, dtype)


def _last_fill_wrong(n, B):
    return n % B


from oracle import block_manager as bm


class _FreeForward(bm.RefBlockManager):
    """Returns a finished request's blocks first block first."""
    def free_seq(self, sid):
        s = self._seq(sid)
        for b in s.table:
            self._release(b)
        del self.seqs[sid]


class _NoEviction(bm.RefBlockManager):
    """Keeps a reused block's old cache entry."""
    def _take(self):
        b = self.free.pop(0)
        self.hash_of[b] = None
        self.ref[b] = 1
        return b


class _CowKeepsRef(bm.RefBlockManager):
    """Copy-on-write without dropping the old block's count."""
    def append(self, sid, tokens):
        s = self._seq(sid)
        shared = [b for b in s.table if self.ref[b] > 1]
        slots, copies = super().append(sid, tokens)
        for src_, _ in copies:
            if src_ in shared:
                self.ref[src_] += 1
        return slots, copies


class _ForkNoRef(bm.RefBlockManager):
    """Fork shares the blocks without counting the new references."""
    def fork(self, parent, child):
        super().fork(parent, child)
        for b in self.seqs[child].table:
            self.ref[b] -= 1


class _HitsUpToFullLength(bm.RefBlockManager):
    """Prefix hits may cover every token, the last one included."""
    def allocate(self, sid, tokens):
        n = len(tokens)
        if n and n % self.B == 0 and self.prefix_caching:
            parent, hits = bm.NONE_HASH, 0
            for i in range(n // self.B):
                parent = bm.block_hash(parent, tokens[i * self.B:(i + 1) * self.B])
                if parent not in self.cache:
                    break
                hits += 1
            if hits == n // self.B:
                cached = super().allocate(sid, tokens)
                return n
        return super().allocate(sid, tokens)


class _HitsPastMiss(bm.RefBlockManager):
    """Keeps looking for hits after the first miss."""
    def allocate(self, sid, tokens):
        if sid in self.seqs:
            raise KeyError(sid)
        n = len(tokens)
        need = -(-n // self.B)
        hits, parent = [], bm.NONE_HASH
        for i in range((n - 1) // self.B if n > 0 else 0):
            h = bm.block_hash(parent, tokens[i * self.B:(i + 1) * self.B])
            if h in self.cache:
                hits.append(self.cache[h])
            parent = h
        in_queue = sum(1 for b in hits if self.ref[b] == 0)
        if len(self.free) - in_queue < need - len(hits):
            raise bm.OutOfBlocks()
        s = bm._Seq()
        for b in hits:
            self._touch(b)
        s.table = hits + [self._take() for _ in range(need - len(hits))]
        s.tokens = list(tokens)
        self.seqs[sid] = s
        self._cache_full(s)
        return len(hits) * self.B


class _CachePartial(bm.RefBlockManager):
    """Also registers the partly filled last block."""
    def _cache_full(self, s):
        super()._cache_full(s)
        if self.prefix_caching and len(s.tokens) % self.B and s.table:
            parent = s.hashes[-1] if s.hashes else bm.NONE_HASH
            h = bm.block_hash(parent, s.tokens[len(s.hashes) * self.B:])
            b = s.table[len(s.hashes)]
            self.cache.setdefault(h, b)
            if self.hash_of[b] is None:
                self.hash_of[b] = h


def _hash_no_parent(parent, tokens):
    return bm.block_hash(bm.NONE_HASH, tokens)


def _copy_blocks_keys_only(kv, pairs, dst=None):
    out = kv if dst is None else dst
    for s, d in pairs:
        out[0, d] = kv[0, s]
    return out


def _prefill_with(positions, causal=True, shift=0):
    """A prefill oracle whose chunk positions or mask bound are planted."""
    def f(query, kv, tables, lens, starts, scale, dtype):
        out = np.zeros(query.shape)
        for s_, L in enumerate(lens):
            r0, r1 = int(starts[s_]), int(starts[s_ + 1])
            k, v = pa.gather_ref(kv, tables[s_], int(L))
            k, v = pa.to_f64(k, dtype), pa.to_f64(v, dtype)
            for i, p in enumerate(positions(int(L), r0, r1)):
                stop = int(L) if not causal else max(0, p + 1 + shift)
                out[r0 + i] = pa.attention_ref(pa.to_f64(query[r0 + i], dtype), k[:stop], v[:stop],
                                               scale)
        return out
    return f


MUTANTS = {
    "prefill_top_left": dict(prefill_attention_ref=_prefill_with(lambda L, r0, r1: range(r1 - r0))),
    "prefill_global_rows": dict(prefill_attention_ref=_prefill_with(
        lambda L, r0, r1: [min(L - 1, r) for r in range(r0, r1)])),
    "prefill_no_mask": dict(prefill_attention_ref=_prefill_with(
        lambda L, r0, r1: range(L - (r1 - r0), L), causal=False)),
    "prefill_mask_excludes_self": dict(prefill_attention_ref=_prefill_with(
        lambda L, r0, r1: range(L - (r1 - r0), L), shift=-1)),
    "prefill_mask_one_ahead": dict(prefill_attention_ref=_prefill_with(
        lambda L, r0, r1: range(L - (r1 - r0), L), shift=1)),
    "bm_free_forward": dict(RefBlockManager=_FreeForward),
    "bm_no_eviction": dict(RefBlockManager=_NoEviction),
    "bm_cow_keeps_ref": dict(RefBlockManager=_CowKeepsRef),
    "bm_fork_no_ref": dict(RefBlockManager=_ForkNoRef),
    "bm_hits_full_length": dict(RefBlockManager=_HitsUpToFullLength),
    "bm_hits_past_miss": dict(RefBlockManager=_HitsPastMiss),
    "bm_cache_partial": dict(RefBlockManager=_CachePartial),
    "hash_no_parent": dict(block_hash=_hash_no_parent),
    "copy_keys_only": dict(copy_blocks_ref=_copy_blocks_keys_only),
    "blocks_floor": dict(blocks_needed=_floor_blocks),
    "slot_swapped_axes": dict(slot_of=_slot_swapped),
    "slot_off_by_one": dict(slot_of=_slot_off_by_one),
    "write_k_v_swapped": dict(write_ref=_write_kv_swapped),
    "gather_wrong_index": dict(gather_ref=_gather_wrong_index),
    "attention_no_scale": dict(attention_ref=_attn_no_scale),
    "attention_head_map": dict(attention_ref=_attn_wrong_head_map),
    "attention_sign": dict(attention_ref=_attn_sign),
    "attention_k_v_transposed": dict(attention_ref=_attn_kv_transposed),
    "attention_unnormalised": dict(attention_ref=_attn_unnormalised),
    "merge_no_exp": dict(merge_ref=_merge_no_exp),
    "merge_no_l": dict(merge_ref=_merge_no_l),
    "page_no_kv_factor": dict(page_bytes=_page_no_kv_factor),
    "widen_wrong_shift": dict(to_f64=_widen_wrong_shift),
    "last_fill_wrong": dict(last_block_fill=_last_fill_wrong),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    ns = pins.namespace(oracle, **MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(ns)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
