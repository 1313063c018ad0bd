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


MUTANTS = {
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
