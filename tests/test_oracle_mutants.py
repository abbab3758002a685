"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one: a dropped term, a wrong index, a transposed operand, a
swapped argument."""
import numpy as np
import pytest

import oracle.paged_attention_ref as ref
from oracle_pins import ALL_PINS


def _attend_no_max(q_h, keys, values, scale):
    s = scale * (keys @ q_h)
    w = np.exp(s)
    return (w @ values) / w.sum()


def _attend_no_scale(q_h, keys, values, scale):
    s = keys @ q_h
    w = np.exp(s - s.max())
    return (w @ values) / w.sum()


def _attend_no_norm(q_h, keys, values, scale):
    s = scale * (keys @ q_h)
    w = np.exp(s - s.max())
    return w @ values


def _attend_keys_as_values(q_h, keys, values, scale):
    s = scale * (keys @ q_h)
    w = np.exp(s - s.max())
    return (w @ keys) / w.sum()


def _attend_wrong_sign(q_h, keys, values, scale):
    s = -scale * (keys @ q_h)
    w = np.exp(s - s.max())
    return (w @ values) / w.sum()


def _token_location_offset(table_row, t, B):
    return np.asarray(table_row)[t // B], (t + 1) % B


def _token_location_block(table_row, t, B):
    return np.asarray(table_row)[t // (2 * B)], t % B


def _token_location_transposed(table_row, t, B):
    return np.asarray(table_row)[t % B], t // B


def _gather_shifted(pool, table_row, num_tokens, block_size, dtype):
    full = ref.__dict__["_orig_gather"](pool, table_row, num_tokens + 1, block_size, dtype)
    return full[1:]


def _gather_short(pool, table_row, num_tokens, block_size, dtype):
    rows = ref.__dict__["_orig_gather"](pool, table_row, num_tokens, block_size, dtype)
    return rows[:-1] if num_tokens > 1 else rows


MUTANTS = {
    "gqa_modulo": ("kv_head_for_query_head", lambda h, hq, hkv: h % hkv),
    "gqa_div_by_kv": ("kv_head_for_query_head", lambda h, hq, hkv: min(h // hkv, hkv - 1)),
    "offset_plus_one": ("token_location", _token_location_offset),
    "wrong_logical_block": ("token_location", _token_location_block),
    "block_offset_swapped": ("token_location", _token_location_transposed),
    "no_max_subtraction": ("attend", _attend_no_max),
    "no_scale": ("attend", _attend_no_scale),
    "no_normalisation": ("attend", _attend_no_norm),
    "keys_as_values": ("attend", _attend_keys_as_values),
    "score_sign": ("attend", _attend_wrong_sign),
    "slot_location_swapped": ("slot_location", lambda s, B: (s % B, s // B)),
    "blocks_floor": ("blocks_for_tokens", lambda T, B: int(T) // int(B)),
    "bf16_shift_15": ("to_float64", lambda a, d: ((a.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
                                                   if d == "bf16" else a.astype(np.float64))),
    "gather_shifted": ("gather_tokens", _gather_shifted),
    "gather_drops_last": ("gather_tokens", _gather_short),
}


def _write_kv_swapped(k_pool, v_pool, k, v, slot_mapping, block_size):
    return ref.__dict__["_orig_write"](k_pool, v_pool, v, k, slot_mapping, block_size)


MUTANTS["write_swaps_k_v"] = ("write_kv", _write_kv_swapped)
MUTANTS["window_one_extra"] = ("window_start", lambda T, W: 0 if W is None else max(0, int(T) - int(W) - 1))
MUTANTS["window_one_short"] = ("window_start", lambda T, W: 0 if W is None else max(0, int(T) - int(W) + 1))
MUTANTS["window_counts_from_start"] = ("window_start", lambda T, W: 0)


def _gather_window_all(pool, table_row, first, num_tokens, block_size, dtype):
    return ref.__dict__["_orig_gather"](pool, table_row, num_tokens, block_size, dtype)


MUTANTS["window_ignored_in_gather"] = ("gather_window", _gather_window_all)
MUTANTS["prefill_excludes_own_key"] = ("causal_keys", lambda p: int(p))
MUTANTS["prefill_sees_next_key"] = ("causal_keys", lambda p: int(p) + 2)
MUTANTS["prefill_rows_from_start"] = ("query_position", lambda T, M, r: int(r))
def _fp8_truncating(y):
    y = np.asarray(y, np.float32)
    out = ref.__dict__["_orig_encode"](y)
    a = np.abs(y.astype(np.float64))
    dec = ref.fp8_e4m3_decode(out)
    # round toward zero instead of to nearest
    return np.where(np.abs(dec) > a, out - 1, out).astype(np.uint8)


def _fp8_ties_up(y):
    y = np.asarray(y, np.float32)
    out = ref.__dict__["_orig_encode"](y)
    a = np.abs(y.astype(np.float64))
    up = ref.__dict__["_orig_encode"]((np.abs(y) * np.float32(1 + 2 ** -20)) * np.sign(y))
    mid = np.abs(ref.fp8_e4m3_decode(out)) != np.abs(ref.fp8_e4m3_decode(up))
    return np.where(mid & (a > 0), up, out).astype(np.uint8)


MUTANTS["fp8_truncates"] = ("fp8_e4m3_encode", _fp8_truncating)
MUTANTS["fp8_ties_away"] = ("fp8_e4m3_encode", _fp8_ties_up)
MUTANTS["fp8_bias_8"] = ("fp8_e4m3_decode", lambda c: ref.__dict__["_orig_decode"](c) / 2.0)
MUTANTS["fp8_scale_ignored"] = ("quantize_fp8", lambda x, d, s: ref.fp8_e4m3_encode(ref.to_float64(x, d).astype(np.float32)))
MUTANTS["prefill_rows_shifted"] = ("query_position", lambda T, M, r: int(T) - int(M) + int(r) - 1)


def _run_pins():
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ref)
        except Exception as e:          # any failure counts: assertion, index, NaN
            failed.append((pin.__name__, type(e).__name__))
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(ref.__dict__, "_orig_gather", ref.gather_tokens)
    monkeypatch.setitem(ref.__dict__, "_orig_write", ref.write_kv)
    monkeypatch.setitem(ref.__dict__, "_orig_encode", ref.fp8_e4m3_encode)
    monkeypatch.setitem(ref.__dict__, "_orig_decode", ref.fp8_e4m3_decode)
    monkeypatch.setattr(ref, attr, fn)
    failed = _run_pins()
    assert failed, f"no pin caught the planted mistake {name!r}"
