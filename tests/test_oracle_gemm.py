"""Pins for the oracle's block-scaled GEMM reference and output rounding (CPU only).

What pins it:
  * brute force: a pure-Python triple loop over dequantized values (each
    element carries its own scale) on the tiny Fprop problem and on small
    Wgrad / grouped problems, to 1e-12 relative;
  * all scales 1: the reference equals numpy's float64 product of the decoded
    operands exactly;
  * linearity in a scale (doubling SA doubles C exactly) and the transpose
    identity (Wgrad with the operands swapped gives C^T);
  * per-group integer partials equal Python-int dot products;
  * block-scale indexing: a scale planted in one (n-block, k-group) cell only
    moves the matching outputs;
  * BF16 output rounding against torch's float32->bfloat16 cast on float32
    inputs, and against hand-made ties;
  * the sampled-entry path equals the full reference.
"""

import numpy as np
import pytest
import torch

from oracle import e4m3, gemm, quant
from workloads import random_fp8_operands, tiny_fprop


def _brute(qa, sa, qb, sb, kind):
    """Triple loop in Python floats: C[m][n] = sum_k (sA*dec a)(sB*dec b)."""
    da, db = e4m3.decode(qa), e4m3.decode(qb)
    m, k = qa.shape
    n = qb.shape[0]
    c = [[0.0] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                g = kk // 128
                sbv = sb[j // 128][g] if kind != gemm.WGRAD else sb[g][j]
                acc += (float(sa[g][i]) * float(da[i, kk])) * (float(sbv) * float(db[j, kk]))
            c[i][j] = acc
    return np.array(c)


def test_tiny_fprop_brute_force():
    d = tiny_fprop()
    qa, sa = quant.quant_1x128(d["a"])
    qb, sb = quant.quant_128x128(d["bt"])
    ref = gemm.gemm_ref(qa, sa, qb, sb, gemm.FPROP, exact_int=True)
    sub = (slice(0, 24), slice(0, 128))                  # 24 rows x all 128 columns
    bf = _brute(qa[sub[0]], sa[:, sub[0]], qb, sb, gemm.FPROP)
    assert gemm.rel_frobenius(bf, ref[sub]) < 1e-13


def test_tiny_fprop_matches_dequantized_product():
    d = tiny_fprop()
    qa, sa = quant.quant_1x128(d["a"])
    qb, sb = quant.quant_128x128(d["bt"])
    ref = gemm.gemm_ref(qa, sa, qb, sb, gemm.FPROP)
    deq = quant.dequant_1x128(qa, sa) @ quant.dequant_128x128(qb, sb).T
    assert gemm.rel_frobenius(ref, deq) < 1e-14
    # and the FP8 product approximates the unquantized one (tile scaling works)
    full = d["a"].astype(np.float64) @ d["bt"].astype(np.float64).T
    assert gemm.rel_frobenius(ref, full) < 0.05


def test_unit_scales_equal_plain_product():
    ops = random_fp8_operands(11, 64, 96, 384)
    ones_a = np.ones_like(ops["sa"])
    ones_b = np.ones_like(ops["sb"])
    ref = gemm.gemm_ref(ops["qa"], ones_a, ops["qb"], ones_b, gemm.FPROP)
    plain = e4m3.decode(ops["qa"]) @ e4m3.decode(ops["qb"]).T
    assert np.array_equal(ref, plain)


def test_linearity_in_scales():
    ops = random_fp8_operands(12, 32, 128, 256)
    ref = gemm.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"])
    ref2 = gemm.gemm_ref(ops["qa"], ops["sa"] * 2, ops["qb"], ops["sb"])
    assert np.array_equal(ref2, 2 * ref)


def test_wgrad_brute_force_and_transpose():
    ops = random_fp8_operands(13, 20, 24, 256, kind="wgrad")
    ref = gemm.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"], gemm.WGRAD)
    bf = _brute(ops["qa"], ops["sa"], ops["qb"], ops["sb"], gemm.WGRAD)
    assert gemm.rel_frobenius(bf, ref) < 1e-13
    swapped = gemm.gemm_ref(ops["qb"], ops["sb"], ops["qa"], ops["sa"], gemm.WGRAD)
    assert gemm.rel_frobenius(swapped, ref.T) < 1e-14


def test_group_partials_match_python_ints():
    ops = random_fp8_operands(14, 6, 5, 300)
    parts = gemm.group_partials(ops["qa"], ops["qb"], exact_int=True)
    parts_f = gemm.group_partials(ops["qa"], ops["qb"], exact_int=False)
    da, db = e4m3.decode(ops["qa"]), e4m3.decode(ops["qb"])
    assert len(parts) == 3
    for g, p in enumerate(parts):
        for i in range(6):
            for j in range(5):
                want = sum(int(da[i, k] * 512) * int(db[j, k] * 512)
                           for k in range(g * 128, min(300, (g + 1) * 128)))
                assert int(p[i, j]) == want and float(parts_f[g][i, j]) == float(want)


def test_block_scale_indexing():
    m, n, k = 16, 256, 384
    ops = random_fp8_operands(15, m, n, k)
    sa = np.ones_like(ops["sa"])
    sb = np.ones_like(ops["sb"])                          # [n/128=2][k/128=3]
    base = gemm.gemm_ref(ops["qa"], sa, ops["qb"], sb)
    sb2 = sb.copy()
    sb2[1, 2] = 4.0                                        # n-block 1, k-group 2
    moved = gemm.gemm_ref(ops["qa"], sa, ops["qb"], sb2)
    assert np.array_equal(moved[:, :128], base[:, :128])
    p2 = e4m3.decode(ops["qa"][:, 256:]) @ e4m3.decode(ops["qb"][128:, 256:]).T
    assert np.array_equal(moved[:, 128:], base[:, 128:] + 3.0 * p2)


def test_grouped_matches_per_group_brute_force():
    rng = np.random.default_rng(16)
    gmap = np.array([0, 0, 2, 1], dtype=np.int32)
    valid = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    qa = valid[rng.integers(0, valid.size, size=(512, 256))]
    sa = rng.uniform(0.5, 2, size=(2, 512)).astype(np.float32)
    qb = valid[rng.integers(0, valid.size, size=(3, 8, 256))]
    sb = rng.uniform(0.5, 2, size=(3, 1, 2)).astype(np.float32)
    ref = gemm.grouped_ref(qa, sa, qb, sb, gmap)
    for t, g in enumerate(gmap):
        rows = slice(t * 128, t * 128 + 3)
        bf = _brute(qa[rows], sa[:, rows], qb[g], sb[g], gemm.FPROP)
        assert gemm.rel_frobenius(bf, ref[rows]) < 1e-13


def test_sampled_entries_equal_full_reference():
    for kind in (gemm.FPROP, gemm.WGRAD):
        ops = random_fp8_operands(17, 64, 256, 512, kind=kind)
        full = gemm.gemm_ref(ops["qa"], ops["sa"], ops["qb"], ops["sb"], kind)
        rng = np.random.default_rng(0)
        r = rng.integers(0, 64, 200)
        c = rng.integers(0, 256, 200)
        ent = gemm.gemm_ref_entries(ops["qa"], ops["sa"], ops["qb"], ops["sb"], r, c, kind)
        assert np.max(np.abs(ent - full[r, c]) / np.abs(full[r, c])) < 1e-13


def test_bf16_rounding_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(18)
    x = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-30, 30, 200_000))).astype(np.float32)
    ours = gemm.round_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_rounding_single_rounding_from_float64():
    # 1 + 2^-8 is the BF16 midpoint of 1 and 1 + 2^-7 (tie -> even -> 1.0);
    # 1 + 2^-8 + 2^-40 is just above it (-> 1 + 2^-7) although float32 would
    # first round it onto the midpoint.
    x = np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -40)])
    assert gemm.round_bf16(x).tolist() == [1.0, 1 + 2.0 ** -7, 1 + 2.0 ** -6, -(1 + 2.0 ** -7)]
    assert gemm.bf16_bits(gemm.round_bf16(np.array([1.0, -2.0]))).tolist() == [0x3F80, 0xC000]


def test_rel_frobenius_closed_form():
    a = np.array([[3.0, 4.0]])
    assert gemm.rel_frobenius(a * 1.0, a) == 0.0
    assert gemm.rel_frobenius(np.array([[3.0, 4.0 + 5e-3]]), a) == pytest.approx(1e-3, rel=1e-12)


def test_nan_codes_rejected():
    qa = np.full((1, 128), 0x7F, np.uint8)
    with pytest.raises(ValueError):
        gemm.gemm_ref(qa, np.ones((1, 1), np.float32), qa, np.ones((1, 1), np.float32))
