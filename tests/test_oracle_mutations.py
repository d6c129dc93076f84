"""Planted mistakes: each test swaps one oracle function for a plausibly
wrong variant (on the CPU only) and checks that at least one pin fails.
This is evidence that the pins in test_oracle_pins.py constrain the oracle
and are not restatements of it."""
import numpy as np
import pytest

import oracle
import oracle.hyb_oracle as ho
import tests.test_oracle_pins as pins

FAIL = (AssertionError, ValueError, IndexError)


def _kept_ties_high(group_bits):
    g = np.asarray(group_bits, dtype=np.uint16)
    key = (g & 0x7FFF).astype(np.int64)
    order = np.argsort(-(key * 4 + np.arange(4)), axis=-1, kind="stable")
    return np.minimum(order[..., 0], order[..., 1]), np.maximum(order[..., 0], order[..., 1])


def _kept_signed(group_bits):
    g = np.asarray(group_bits, dtype=np.uint16).view(np.int16).astype(np.int64)
    order = np.argsort(-(g * 4 + (3 - np.arange(4))), axis=-1, kind="stable")
    return np.minimum(order[..., 0], order[..., 1]), np.maximum(order[..., 0], order[..., 1])


def _nibble_swapped(i0, i1, meta):
    i0 = np.asarray(i0, dtype=np.int64)
    i1 = np.asarray(i1, dtype=np.int64)
    if meta == "idx2":
        return (i1 | (i0 << 2)).astype(np.uint8)
    return ((1 << i0) | (1 << i1)).astype(np.uint8)


def _value_index_j_swapped(s, r, g, j, b1, b2):
    return (s * (b1 * b2 // 2) + (r // 16) * 8 * b2 + (g // 16) * 512
            + ((g % 16) // 4) * 128 + (r % 16) * 8 + (g % 4) * 2 + (1 - j))


def _meta_word_blocks_outer(s, r, g, b1, b2):
    return (s * (b1 * b2 // 16) + (r // 16) * b2
            + (g // 16) * 64 + ((g % 16) // 4) * 16 + r % 16)


def _dense_index_rows_cols(s, r, c, b1, b2):
    return (s * b1 * b2 + (r // 16) * 16 * b2 + (c // 32) * 512
            + (r % 16) * 32 + c % 32)


def _ref_transposed(wp_bits, x_bits, dtype):
    w = ho.widen(wp_bits, dtype)
    x = ho.widen(np.atleast_2d(np.asarray(x_bits, dtype=np.uint16)), dtype)
    return x @ w, np.abs(x) @ np.abs(w)


def _ref_reversed_rows(wp_bits, x_bits, dtype):
    w = ho.widen(wp_bits, dtype)
    x = ho.widen(np.atleast_2d(np.asarray(x_bits, dtype=np.uint16)), dtype)
    return (x @ w.T)[:, ::-1], np.abs(x) @ np.abs(w).T


def _ref_drop_last(wp_bits, x_bits, dtype):
    w = ho.widen(wp_bits, dtype)[:, :-1]
    x = ho.widen(np.atleast_2d(np.asarray(x_bits, dtype=np.uint16)), dtype)[:, :-1]
    return x @ w.T, np.abs(x) @ np.abs(w).T


def _ref_signed_bound(wp_bits, x_bits, dtype):
    w = ho.widen(wp_bits, dtype)
    x = ho.widen(np.atleast_2d(np.asarray(x_bits, dtype=np.uint16)), dtype)
    return x @ w.T, np.abs(x @ w.T)


def _prune_keeps_three(w_bits, tile_map, b1, b2, meta="idx2"):
    w = np.asarray(w_bits, dtype=np.uint16)
    n, k = w.shape
    tn_count, tk_count = ho.check_shape(n, k, b1, b2)
    tmap = np.asarray(tile_map, dtype=np.uint8).reshape(tn_count, tk_count)
    out = w.copy()
    for tn in range(tn_count):
        for tk in range(tk_count):
            if tmap[tn, tk]:
                g = out[tn * b1:(tn + 1) * b1, tk * b2:(tk + 1) * b2].reshape(b1, b2 // 4, 4)
                key = (g & 0x7FFF).astype(np.int64)
                low = np.argmin(key * 4 + np.arange(4), axis=-1)
                np.put_along_axis(g, low[..., None], np.uint16(0), axis=-1)
    return out


@pytest.mark.parametrize("name,func", [("kept_positions", _kept_ties_high),
                                       ("kept_positions", _kept_signed),
                                       ("nibble", _nibble_swapped)])
def test_group_rule_mutations_caught(monkeypatch, golden_dir, name, func):
    monkeypatch.setattr(ho, name, func)
    monkeypatch.setattr(oracle, name, func)
    with pytest.raises(FAIL):
        pins.test_golden_groups(golden_dir)


@pytest.mark.parametrize("name,func", [("value_index", _value_index_j_swapped),
                                       ("meta_word_index", _meta_word_blocks_outer),
                                       ("dense_index", _dense_index_rows_cols)])
def test_layout_mutations_caught(monkeypatch, name, func):
    monkeypatch.setattr(ho, name, func)
    with pytest.raises(FAIL):
        pins.test_layout_restatement(32, 128, "idx2")


@pytest.mark.parametrize("func", [_ref_transposed, _ref_reversed_rows, _ref_drop_last, _ref_signed_bound])
def test_reference_mutations_caught(monkeypatch, func):
    monkeypatch.setattr(ho, "ref_matmul", func)
    monkeypatch.setattr(oracle, "ref_matmul", func)
    with pytest.raises(FAIL):
        pins.test_ref_matmul_fsum("bf16")


def test_prune_mutation_caught(monkeypatch):
    monkeypatch.setattr(ho, "prune", _prune_keeps_three)
    monkeypatch.setattr(oracle, "prune", _prune_keeps_three)
    with pytest.raises(FAIL):
        pins.test_invariants(3, "idx2")
    with pytest.raises(FAIL):
        pins.test_invariants(3, "mask8")


def _lowrank_u_transposed(wp_bits, x_bits, t, u_bits, dtype):
    y, s = ho.ref_matmul(wp_bits, x_bits, dtype)
    tt = np.atleast_2d(np.asarray(t, dtype=np.float64))
    uu = ho.widen(np.atleast_2d(np.asarray(u_bits, dtype=np.uint16)), dtype)
    uu = uu.T.reshape(uu.shape) if uu.shape[0] != uu.shape[1] else uu.T
    return y + tt @ uu.T, s + np.abs(tt) @ np.abs(uu).T


def _lowrank_dropped(wp_bits, x_bits, t, u_bits, dtype):
    return ho.ref_matmul(wp_bits, x_bits, dtype)


def _lowrank_sign(wp_bits, x_bits, t, u_bits, dtype):
    y, s = ho.ref_matmul(wp_bits, x_bits, dtype)
    tt = np.atleast_2d(np.asarray(t, dtype=np.float64))
    uu = ho.widen(np.atleast_2d(np.asarray(u_bits, dtype=np.uint16)), dtype)
    return y - tt @ uu.T, s + np.abs(tt) @ np.abs(uu).T


def _lowrank_last_rank_dropped(wp_bits, x_bits, t, u_bits, dtype):
    y, s = ho.ref_matmul(wp_bits, x_bits, dtype)
    tt = np.atleast_2d(np.asarray(t, dtype=np.float64))[:, :-1]
    uu = ho.widen(np.atleast_2d(np.asarray(u_bits, dtype=np.uint16)), dtype)[:, :-1]
    return y + tt @ uu.T, s + np.abs(tt) @ np.abs(uu).T


@pytest.mark.parametrize("func", [_lowrank_u_transposed, _lowrank_dropped, _lowrank_sign,
                                  _lowrank_last_rank_dropped])
def test_lowrank_mutations_caught(monkeypatch, golden_dir, func):
    monkeypatch.setattr(ho, "ref_lowrank", func)
    monkeypatch.setattr(oracle, "ref_lowrank", func)
    caught = 0
    for pin in (lambda: pins.test_ref_lowrank_golden(golden_dir), pins.test_ref_lowrank_loops_and_special_cases):
        try:
            pin()
        except FAIL:
            caught += 1
    assert caught >= 1


# ------------------------------------------------------------------ 4:8 ----

def _kept_nm_ties_high(group_bits, keep):
    g = np.asarray(group_bits, dtype=np.uint16)
    size = g.shape[-1]
    key = (g & 0x7FFF).astype(np.int64)
    order = np.argsort(-(key * size + np.arange(size)), axis=-1, kind="stable")
    return np.sort(order[..., :keep], axis=-1)


def _kept_nm_per_half(group_bits, keep):
    """Top keep/2 of each half instead of top keep of the whole group."""
    g = np.asarray(group_bits, dtype=np.uint16)
    size = g.shape[-1]
    h = size // 2
    key = (g & 0x7FFF).astype(np.int64)
    out = []
    for lo in (0, h):
        k = key[..., lo:lo + h]
        order = np.argsort(-(k * h + (h - 1 - np.arange(h))), axis=-1, kind="stable")
        out.append(order[..., :keep // 2] + lo)
    return np.sort(np.concatenate(out, axis=-1), axis=-1)


def _mask8_reversed(positions):
    p = np.asarray(positions, dtype=np.int64)
    return np.bitwise_or.reduce(np.left_shift(1, 7 - p), axis=-1).astype(np.uint8)


def _value_index8_reversed(s, r, h, j, b1, b2):
    return (s * (b1 * b2 // 2) + (r // 16) * 8 * b2 + (h // 8) * 512
            + ((h % 8) // 2) * 128 + (r % 16) * 8 + (h % 2) * 4 + (3 - j))


def _value_index8_groups_swapped(s, r, h, j, b1, b2):
    return (s * (b1 * b2 // 2) + (r // 16) * 8 * b2 + (h // 8) * 512
            + ((h % 8) // 2) * 128 + (r % 16) * 8 + (1 - h % 2) * 4 + j)


@pytest.mark.parametrize("name,func", [("kept_positions_nm", _kept_nm_ties_high),
                                       ("kept_positions_nm", _kept_nm_per_half),
                                       ("mask8", _mask8_reversed)])
def test_4of8_rule_mutations_caught(monkeypatch, golden_dir, name, func):
    monkeypatch.setattr(ho, name, func)
    monkeypatch.setattr(oracle, name, func)
    with pytest.raises(FAIL):
        pins.test_golden_groups_4of8(golden_dir)


@pytest.mark.parametrize("func", [_value_index8_reversed, _value_index8_groups_swapped])
def test_4of8_layout_mutations_caught(monkeypatch, func):
    monkeypatch.setattr(ho, "value_index8", func)
    with pytest.raises(FAIL):
        pins.test_layout_restatement(32, 128, "mask8")


def test_4of8_per_half_rule_caught_by_magnitude_pin(monkeypatch):
    monkeypatch.setattr(ho, "kept_positions_nm", _kept_nm_per_half)
    monkeypatch.setattr(oracle, "kept_positions_nm", _kept_nm_per_half)
    with pytest.raises(FAIL):
        pins.test_4of8_keeps_at_least_the_2of4_magnitude()



# ------------------------------------------------ value and acceptance pins -

def _widen_swapped(bits, dtype):
    other = {"f16": "bf16", "bf16": "f16"}.get(dtype, dtype)
    b = np.asarray(bits, dtype=np.uint16)
    if other == "f16":
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _widen_f16_flush(bits, dtype):
    """fp16 subnormals flushed to zero (a plausible decoder shortcut)."""
    b = np.asarray(bits, dtype=np.uint16)
    v = _widen_swapped(b, "bf16" if dtype == "f16" else "f16")
    if dtype == "f16":
        v = np.where((b & 0x7C00) == 0, np.copysign(0.0, v), v)
    return v


@pytest.mark.parametrize("func", [_widen_swapped, _widen_f16_flush])
def test_widen_mutations_caught(monkeypatch, golden_dir, func):
    monkeypatch.setattr(ho, "widen", func)
    monkeypatch.setattr(oracle, "widen", func)
    with pytest.raises(FAIL):
        pins.test_widen_golden(golden_dir, "f16", "f16_values.txt")


def test_widen_swap_caught_by_f16_product(monkeypatch):
    monkeypatch.setattr(ho, "widen", _widen_swapped)
    monkeypatch.setattr(oracle, "widen", _widen_swapped)
    with pytest.raises(FAIL):
        pins.test_ref_matmul_integers_exact_f16()


def _within_strict(y, y_ref, s, rel=2e-3, extra=0.0):
    return np.abs(np.asarray(y, dtype=np.float64) - y_ref) < rel * s + extra


def _within_rel_ignored(y, y_ref, s, rel=2e-3, extra=0.0):
    return np.abs(np.asarray(y, dtype=np.float64) - y_ref) <= 2e-3 * s + extra


@pytest.mark.parametrize("func", [_within_strict, _within_rel_ignored])
def test_within_bound_mutations_caught(monkeypatch, func):
    monkeypatch.setattr(ho, "within_bound", func)
    monkeypatch.setattr(oracle, "within_bound", func)
    with pytest.raises(FAIL):
        pins.test_within_bound_cases()


def _ref_rows_all(wp_bits, x_bits, dtype, rows):
    return ho.ref_matmul(wp_bits, x_bits, dtype)


def _ref_rows_sorted(wp_bits, x_bits, dtype, rows):
    return ho.ref_matmul(np.asarray(wp_bits)[np.sort(np.asarray(rows))], x_bits, dtype)


@pytest.mark.parametrize("func", [_ref_rows_all, _ref_rows_sorted])
def test_ref_rows_mutations_caught(monkeypatch, func):
    monkeypatch.setattr(ho, "ref_rows", func)
    monkeypatch.setattr(oracle, "ref_rows", func)
    with pytest.raises(FAIL):
        pins.test_ref_rows_selects_rows()
