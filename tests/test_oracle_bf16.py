"""Pins of the BF16 input widening, on the CPU.

Every BF16 quantizer test feeds the oracle through ``oracle.quant.bf16_bits_to_f32``
and the seeded inputs through ``workloads.bf16_bits_as_f32``; the quantizer rule
reads x "widened exactly from BF16" (a BF16 value is the top half of the float32
with the same sign, exponent and leading 7 mantissa bits).  Both functions are
checked here against things other than themselves:
  * torch's own bfloat16 -> float32 cast, for all 65,536 bit patterns;
  * values fixed by the BF16 field layout (sign 1, exponent 8, mantissa 7 bits,
    bias 127), written out by hand;
  * the nearest-even float32 -> BF16 cast the input generator uses, which must
    give every non-NaN pattern back unchanged.
"""

import numpy as np
import pytest
import torch

from oracle.quant import bf16_bits_to_f32
from workloads import bf16_bits_as_f32, to_bf16_bits

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
WIDEN = [bf16_bits_to_f32, bf16_bits_as_f32]


def _torch_widen(bits):
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float32).numpy()


@pytest.mark.parametrize("widen", WIDEN, ids=["oracle", "workloads"])
def test_every_pattern_matches_torch_cast(widen):
    got = widen(ALL)
    ref = _torch_widen(ALL)
    assert got.dtype == np.float32 and got.shape == ALL.shape
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    # identical float32 bits for every non-NaN pattern (signed zeros, subnormals, infinities included)
    assert np.array_equal(got.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])
    # NaN patterns keep their sign and payload: the BF16 bits are the top half
    assert np.array_equal(got.view(np.uint32)[nan] >> 16, ALL[nan].astype(np.uint32))


@pytest.mark.parametrize("widen", WIDEN, ids=["oracle", "workloads"])
def test_field_layout_values(widen):
    # (bits, value) from the BF16 definition: (-1)^s * 2^(e-127) * (1 + m/128), subnormal 2^-126 * m/128
    cases = [
        (0x0000, 0.0), (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0xC040, -3.0),
        (0x3F00, 0.5), (0x3FC0, 1.5), (0x4120, 10.0), (0x43E0, 448.0), (0x3C00, 2.0 ** -7),
        (0x0080, 2.0 ** -126), (0x0001, 2.0 ** -133), (0x007F, 127 * 2.0 ** -133),
        (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127), (0x7F80, np.inf), (0xFF80, -np.inf),
    ]
    bits = np.array([c[0] for c in cases], dtype=np.uint16)
    got = widen(bits).astype(np.float64)
    assert np.array_equal(got, np.array([c[1] for c in cases], dtype=np.float64))
    neg_zero = widen(np.array([0x8000], dtype=np.uint16))
    assert neg_zero[0] == 0.0 and np.signbit(neg_zero[0])


@pytest.mark.parametrize("widen", WIDEN, ids=["oracle", "workloads"])
def test_generator_cast_gives_every_pattern_back(widen):
    vals = widen(ALL)
    keep = ~np.isnan(vals)
    assert np.array_equal(to_bf16_bits(vals[keep]), ALL[keep])


def test_widening_is_monotone_on_positive_finite_patterns():
    # BF16 ordering of positive finite patterns is the integer ordering of their bits
    pos = ALL[:0x7F80]
    v = bf16_bits_to_f32(pos).astype(np.float64)
    assert np.all(np.diff(v) > 0)
