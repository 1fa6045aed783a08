"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin fails.

Each case swaps one oracle function for a subtly wrong version with pytest's
monkeypatch and runs the pin that is meant to catch it.
"""

import numpy as np
import pytest

from oracle import e4m3, gemm, quant
import tests.test_oracle_bf16 as pins_bf16
import tests.test_oracle_e4m3 as pins_e4m3
import tests.test_oracle_gemm as pins_gemm
import tests.test_oracle_quant as pins_quant


def _encode_ties_away(v):
    v = np.asarray(v, np.float32)
    a = np.minimum(np.abs(v).astype(np.float64), 448.0)
    mags = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    lo = np.clip(np.searchsorted(mags, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    code = np.where(a - mags[lo] < mags[hi] - a, lo, hi).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def _scales_inverted(amax, mode):
    s, inv = ORIG_SCALES(amax, mode)
    return inv, s


def _scales_pow2_round_down(amax, mode):
    s, inv = ORIG_SCALES(amax, mode)
    if mode == quant.MODE_POW2:
        return (s / 2).astype(np.float32), (inv * 2).astype(np.float32)
    return s, inv


def _sigma_b_transposed(sb, kind, g, n_idx):
    sb = np.asarray(sb, np.float64)
    if kind == gemm.WGRAD:
        return sb[g, n_idx]
    return sb[(n_idx // 128) % sb.shape[0], g % sb.shape[1]] if sb.shape[0] == 1 else sb[g % sb.shape[0], (n_idx // 128) % sb.shape[1]]


ORIG_SCALES = quant.scales_from_amax


def test_ties_away_from_zero_is_caught(monkeypatch):
    monkeypatch.setattr(e4m3, "encode", _encode_ties_away)
    with pytest.raises(AssertionError):
        pins_e4m3.test_golden_encode_cases()
    with pytest.raises(AssertionError):
        pins_e4m3.test_encode_around_every_midpoint_matches_torch()


def test_inverted_scale_is_caught(monkeypatch):
    monkeypatch.setattr(quant, "scales_from_amax", _scales_inverted)
    with pytest.raises(AssertionError):
        pins_quant.test_maxabs_maps_each_tile_max_to_448()


def test_pow2_rounded_down_is_caught(monkeypatch):
    monkeypatch.setattr(quant, "scales_from_amax", _scales_pow2_round_down)
    with pytest.raises(AssertionError):
        pins_quant.test_pow2_scale_properties()


def test_transposed_block_scale_index_is_caught(monkeypatch):
    monkeypatch.setattr(gemm, "_sigma_b", _sigma_b_transposed)
    with pytest.raises((AssertionError, IndexError)):
        pins_gemm.test_block_scale_indexing()


def test_dropped_integer_rescale_is_caught(monkeypatch):
    monkeypatch.setattr(gemm, "_PAIR_SCALE", 2.0 ** -9)
    with pytest.raises(AssertionError):
        pins_gemm.test_unit_scales_equal_plain_product()


def _requant_without_dequant(q, s, mode=quant.MODE_POW2):
    return quant.quant_128x1(e4m3.decode(np.asarray(q, np.uint8)).astype(np.float32), mode)


def _requant_wrong_group_scale(q, s, mode=quant.MODE_POW2):
    s = np.asarray(s, np.float32)
    return ORIG_REQUANT(q, np.roll(s, 1, axis=0), mode)


ORIG_REQUANT = quant.requant_1x128_to_128x1


def test_requant_without_dequantization_is_caught(monkeypatch):
    monkeypatch.setattr(quant, "requant_1x128_to_128x1", _requant_without_dequant)
    with pytest.raises(AssertionError):
        pins_quant.test_requant_scale_covariance(quant.MODE_POW2)


def test_requant_with_another_groups_scale_is_caught(monkeypatch):
    monkeypatch.setattr(quant, "requant_1x128_to_128x1", _requant_wrong_group_scale)
    with pytest.raises(AssertionError):
        pins_quant.test_requant_error_bound_against_source(quant.MODE_POW2)


def _widen_shift_15(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(15)).view(np.float32)


def _widen_without_shift(bits):
    # the pattern left in the low half of the float32 word
    return np.asarray(bits, dtype=np.uint16).astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("mutant", [_widen_shift_15, _widen_without_shift], ids=["shift15", "no-shift"])
def test_wrong_bf16_widening_is_caught(mutant):
    with pytest.raises(AssertionError):
        pins_bf16.test_every_pattern_matches_torch_cast(mutant)
    with pytest.raises(AssertionError):
        pins_bf16.test_field_layout_values(mutant)
