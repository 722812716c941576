"""Planted mistakes in the oracle must each be caught by at least one pin.

Every mutant replaces one of the oracle's named steps with a plausible wrong version (a dropped term,
a wrong sign or index, a transposed or swapped operand, an off-by-one).  All mutations happen on the
CPU, in the oracle only.
"""

import numpy as np
import pytest

import oracle.paged_kv as O
from oracle_pins import ALL_PINS


def _orig(name):
    return getattr(O, name)


def _attend_head_factory(kind):
    def attend_head(qh, kh, vh, mask, scale):
        if kind == "no_scale":
            s = qh @ kh.T
        elif kind == "sqrt_scale":
            s = (qh @ kh.T) * np.sqrt(scale)
        elif kind == "keys_as_values":
            s = (qh @ kh.T) * scale
            return O.softmax_rows(np.where(mask, s, -np.inf)) @ kh
        elif kind == "values_as_keys":
            s = (qh @ vh.T) * scale
        elif kind == "mask_ignored":
            return O.softmax_rows((qh @ kh.T) * scale) @ vh
        elif kind == "mask_after_softmax":
            p = O.softmax_rows((qh @ kh.T) * scale)
            return np.where(mask, p, 0.0) @ vh
        else:
            raise AssertionError(kind)
        return O.softmax_rows(np.where(mask, s, -np.inf)) @ vh
    return attend_head


def _gather_reversed(pool, table_row, context_len):
    bs = pool.shape[1]
    nb = -(-context_len // bs)
    if nb == 0:
        return pool[:0, 0]
    return np.concatenate([pool[int(table_row[j])] for j in reversed(range(nb))], axis=0)[:context_len]


def _gather_first_block_only(pool, table_row, context_len):
    bs = pool.shape[1]
    nb = -(-context_len // bs)
    if nb == 0:
        return pool[:0, 0]
    return np.concatenate([pool[int(table_row[0])] for _ in range(nb)], axis=0)[:context_len]


def _kv_write_no_skip(k_pool, v_pool, k_new, v_new, slot_mapping):
    k_out, v_out = k_pool.copy(), v_pool.copy()
    bs = k_pool.shape[1]
    for t in range(len(slot_mapping)):
        blk, off = divmod(int(slot_mapping[t]), bs)
        k_out[blk, off] = k_new[t]
        v_out[blk, off] = v_new[t]
    return k_out, v_out


def _kv_write_k_into_both(k_pool, v_pool, k_new, v_new, slot_mapping):
    return _orig_kv_write(k_pool, v_pool, k_new, k_new, slot_mapping)


_orig_kv_write = O.kv_write

MUTANTS = {
    "kv_head_modulo": ("kv_head_of", lambda h, g: h % g),
    "kv_head_last_in_group_shifted": ("kv_head_of", lambda h, g: h // g + (1 if g > 1 and h % g == g - 1 else 0)),
    "causal_top_left": ("last_visible_key", lambda i, n, L: i),
    "causal_minus_one": ("last_visible_key", lambda i, n, L: L - n + i - 1),
    "causal_plus_one": ("last_visible_key", lambda i, n, L: L - n + i + 1),
    "blocks_floor": ("logical_block_count", lambda L, bs: L // bs),
    "slot_swapped": ("slot_to_block_offset", lambda slot, bs: (slot % bs, slot // bs)),
    "slot_offset_shift": ("slot_to_block_offset", lambda slot, bs: (slot // bs, (slot + 1) % bs)),
    "gather_reversed": ("gather_sequence", _gather_reversed),
    "gather_first_block": ("gather_sequence", _gather_first_block_only),
    "softmax_unnormalised": ("softmax_rows", lambda s: np.exp(s - np.max(s, axis=1, keepdims=True))),
    "softmax_wrong_axis": ("softmax_rows", lambda s: (lambda e: e / np.sum(e, axis=0, keepdims=True))(np.exp(s - np.max(s, axis=1, keepdims=True)))),
    "no_scale": ("attend_head", _attend_head_factory("no_scale")),
    "sqrt_scale": ("attend_head", _attend_head_factory("sqrt_scale")),
    "keys_as_values": ("attend_head", _attend_head_factory("keys_as_values")),
    "values_as_keys": ("attend_head", _attend_head_factory("values_as_keys")),
    "mask_ignored": ("attend_head", _attend_head_factory("mask_ignored")),
    "mask_after_softmax": ("attend_head", _attend_head_factory("mask_after_softmax")),
    "scores_transposed_sign": ("head_scores", lambda qh, kh, scale: -(qh @ kh.T) * scale),
    "write_ignores_skip": ("kv_write", _kv_write_no_skip),
    "write_k_into_v": ("kv_write", _kv_write_k_into_both),
    "bf16_shift_15": ("to_float64", lambda x, dt: (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 15).view(np.float32).astype(np.float64) if dt == "bf16" else np.asarray(x, np.float32).astype(np.float64)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure of a pin counts as catching the mutant
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
