"""Quantization-error study of the scaling rules (CPU, oracle only).

Checks the conclusions the study table in the design notes rests on, on small
seeded tensors of the workloads' distributions:
  * every rule stays inside the E4M3 rounding bound (3 mantissa bits: each
    element in the normal range is off by at most 2^-4 of itself, so the
    relative Frobenius error is at most 2^-4 unless values underflow or clip);
  * on outlier-bearing activations 1x128 max-abs tiles beat a per-tensor
    scale: each tile's max-abs lands exactly on 448, and the large entries
    dominate the error norm;
  * power-of-two scales give up that exact top code and cost accuracy;
  * a delayed (history) per-tensor scale clips a spike the history has not
    seen, while the online tile scale absorbs it.
"""

import numpy as np

from oracle import quant, study
from workloads import add_outliers, normal_f32


def _act(seed, shape=(512, 1024), frac=0.001, factor=50.0):
    rng = np.random.default_rng(seed)
    return add_outliers(rng, normal_f32(rng, shape, 1.0), frac, factor)


def test_all_rules_within_e4m3_rounding_bound():
    x = _act(1)
    for mode in (quant.MODE_MAXABS, quant.MODE_POW2):
        for fn in (study.per_tensor, study.fine_1x128, study.fine_128x128):
            q, _, d = fn(x, mode)
            assert study.rel_error(d, x) <= 2.0 ** -4, (fn.__name__, mode)


def test_tiles_beat_per_tensor_on_outlier_activations():
    x = _act(2)
    e_tensor = study.rel_error(study.per_tensor(x)[2], x)
    e_tile = study.rel_error(study.fine_1x128(x, quant.MODE_MAXABS)[2], x)
    assert e_tile < 0.7 * e_tensor, (e_tile, e_tensor)


def test_pow2_costs_accuracy_against_maxabs_tiles():
    x = _act(3)
    e_max = study.rel_error(study.fine_1x128(x, quant.MODE_MAXABS)[2], x)
    e_p2 = study.rel_error(study.fine_1x128(x, quant.MODE_POW2)[2], x)
    assert e_max < e_p2 <= 2.0 ** -4


def test_delayed_scaling_clips_an_unseen_spike():
    rng = np.random.default_rng(4)
    base = _act(5, (256, 512))
    xs = []
    for t in range(6):
        x = base[rng.permutation(base.shape[0])].copy()
        if t == 4:
            flat = x.reshape(-1)
            idx = rng.choice(flat.size, 16, replace=False)
            flat[idx] = np.float32(4.0) * np.max(np.abs(base))
        xs.append(x)
    errs, clipped = study.delayed_sequence(xs, history=3)
    online = study.rel_error(study.fine_1x128(xs[4], quant.MODE_MAXABS)[2], xs[4])
    assert clipped[4] > 0 and all(c == 0 for i, c in enumerate(clipped) if i != 4)
    assert errs[4] > 10 * online
    assert max(errs[:4] + errs[5:]) <= 2.0 ** -4


def test_underflow_fraction_closed_form():
    # nonzero inputs whose code is +0 (0x00) or -0 (0x80) over all nonzero inputs;
    # zero inputs do not count, whatever their code
    x = np.array([1.0, -1.0, 2.0, 3.0, 0.0, 0.0, -5.0, 7.0], np.float32)
    q = np.array([0x00, 0x80, 0x01, 0x7E, 0x00, 0x80, 0x81, 0xFE], np.uint8)
    assert study.underflow_fraction(q, x) == 2 / 6
    assert study.underflow_fraction(np.array([0x08, 0x88], np.uint8), np.array([1.0, -1.0], np.float32)) == 0.0
    assert study.underflow_fraction(np.array([0x80], np.uint8), np.array([-1e-30], np.float32)) == 1.0


def test_underflow_fraction_counts_values_below_half_the_smallest_subnormal():
    # with unit scales, |x| <= 2^-10 (half of E4M3's smallest subnormal 2^-9) rounds to zero
    # (the tie 2^-10 goes to the even code 0); 2^-9 and above does not
    x = np.array([2.0 ** -11, -(2.0 ** -10), 2.0 ** -9, 1.0], np.float32)
    q, _ = study.quant_with_scale(x, np.float32(1.0), np.float32(1.0))
    assert study.underflow_fraction(q, x) == 2 / 4
