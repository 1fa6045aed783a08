"""Pins for the oracle's E4M3FN codec (CPU only).

Pinned against: torch's independent float8_e4m3fn implementation (decode of
every byte, encode of every finite BF16 pattern in range and of every value
around each rounding midpoint), the round trip of representable values, and
hand-worked cases in tests/golden/worked_examples.json.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _torch_encode(v_f32):
    return torch.from_numpy(np.ascontiguousarray(v_f32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _f32(hexstr):
    return np.array([int(hexstr, 16)], dtype=np.uint32).view(np.float32)


def test_decode_matches_torch_for_every_byte():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    ours = e4m3.decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])


def test_format_constants():
    fi = torch.finfo(torch.float8_e4m3fn)
    assert e4m3.E4M3_MAX == fi.max == 448.0
    assert e4m3.decode(np.array([0x08], np.uint8))[0] == fi.smallest_normal == 2.0 ** -6
    assert e4m3.decode(np.array([0x01], np.uint8))[0] == 2.0 ** -9


def test_encode_every_bf16_pattern_in_range_matches_torch():
    bits = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    assert np.array_equal(e4m3.encode(v), _torch_encode(v))


def test_encode_around_every_midpoint_matches_torch():
    mags = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    mids = (0.5 * (mags[:-1] + mags[1:])).astype(np.float32)     # exact in float32
    assert np.array_equal(mids.astype(np.float64), 0.5 * (mags[:-1] + mags[1:]))
    pts = np.concatenate([mags.astype(np.float32), mids])
    ulp_steps = np.arange(-4, 5, dtype=np.int64)
    bits = pts.view(np.int32).astype(np.int64)[:, None] + ulp_steps[None, :]
    v = bits.reshape(-1)
    v = v[v >= 0].astype(np.int32).view(np.float32)
    v = v[np.abs(v) <= 448.0]
    v = np.concatenate([v, -v])
    assert np.array_equal(e4m3.encode(v), _torch_encode(v))


def test_encode_random_float32_matches_torch():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 0x43E00001, size=2_000_000, dtype=np.int64).astype(np.int32)
    v = bits.view(np.float32)
    v = np.where(rng.random(v.size) < 0.5, -v, v).astype(np.float32)
    assert np.array_equal(e4m3.encode(v), _torch_encode(v))


def test_round_trip_of_representable_values():
    codes = np.array([c for c in range(256) if c not in e4m3.NAN_CODES], dtype=np.uint8)
    vals = e4m3.decode(codes).astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes)


def test_saturation_and_sign():
    v = np.array([448.0, 449.0, 463.99, 464.0, 470.0, 1e30, -1e30, -449.0], np.float32)
    assert e4m3.encode(v).tolist() == [0x7E] * 6 + [0xFE, 0xFE]


def test_non_finite_rejected():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.inf], np.float32))
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan], np.float32))


def test_golden_encode_cases():
    cases = json.load(open(GOLDEN))["encode_cases"]
    for c in cases:
        got = int(e4m3.encode(_f32(c["x"]))[0])
        assert got == int(c["code"], 16), c["why"]
