"""Property-based pins of the oracle (CPU only, hypothesis, derandomized).

The fixed-seed pins in test_oracle_quant.py and test_oracle_gemm.py are
widened here to generated cases: every shape from one element up to ragged
multi-group tensors, every finite E4M3 code, and group magnitudes across the
whole float32 range.  Nothing here retypes the oracle's formulas; each case
checks a property that the definition fixes:
  * GEMM group partials: the exact integer sum of dec(a)*dec(b)*2^18 over each
    128-deep K-group (Python integers), for any K, in both the int64 and the
    float64 form;
  * 1x128 max-abs: a tile whose max-abs clears the floor 448*2^-126 has
    max |dec(q)| == 448; below the floor the scale is the floor's and every
    code stays below 448;
  * 1x128 pow2: s is an integral power of two with a/s in (224, 448]
    (a the floored max-abs), so the largest code lies in [224, 448];
  * both modes: every element is within half an E4M3 step (at the scaled
    magnitude) plus the two-rounding term of its original value; signs are
    kept;
  * 128x128 blocks: the same max-abs property per block, on ragged blocks.
"""

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import e4m3, gemm, quant

SETTINGS = settings(derandomize=True, max_examples=60, deadline=None)
FLOOR = 448.0 * 2.0 ** -126
FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _codes(rng, shape):
    return FINITE_CODES[rng.integers(0, FINITE_CODES.size, size=shape)]


@SETTINGS
@given(m=st.integers(1, 4), n=st.integers(1, 4), k=st.integers(1, 300), seed=st.integers(0, 2 ** 32 - 1))
def test_group_partials_are_exact_integer_sums(m, n, k, seed):
    rng = np.random.default_rng(seed)
    qa, qb = _codes(rng, (m, k)), _codes(rng, (n, k))
    da = [[int(v * 512) for v in row] for row in e4m3.decode(qa)]      # dec * 2^9 is an integer
    db = [[int(v * 512) for v in row] for row in e4m3.decode(qb)]
    parts = gemm.group_partials(qa, qb, exact_int=True)
    parts_f = gemm.group_partials(qa, qb, exact_int=False)
    assert len(parts) == -(-k // 128)
    for g in range(len(parts)):
        ks = range(g * 128, min(k, (g + 1) * 128))
        for i in range(m):
            for j in range(n):
                want = sum(da[i][t] * db[j][t] for t in ks)
                assert int(parts[g][i, j]) == want
                assert float(parts_f[g][i, j]) == float(want)


def _row_groups(draw_exps, rng, cols):
    """One row of `cols` float32 values whose 128-wide groups each have their
    own magnitude 2^e (e drawn per group)."""
    x = rng.standard_normal(cols)
    for g, e in enumerate(draw_exps):
        x[g * 128:(g + 1) * 128] *= 2.0 ** e
    return x.astype(np.float32)


def _groups(cols):
    return -(-cols // 128)


@SETTINGS
@given(cols=st.integers(1, 400), seed=st.integers(0, 2 ** 32 - 1),
       exps=st.lists(st.integers(-150, 120), min_size=4, max_size=4),
       mode=st.sampled_from([quant.MODE_MAXABS, quant.MODE_POW2]))
def test_1x128_tile_properties_across_the_float32_range(cols, seed, exps, mode):
    rng = np.random.default_rng(seed)
    x = _row_groups(exps[:_groups(cols)], rng, cols)[None, :]
    if not np.all(np.isfinite(x)):
        return
    q, s = quant.quant_1x128(x, mode)
    assert q.shape == (1, cols) and s.shape == (_groups(cols), 1)
    d = e4m3.decode(q)[0]
    xs = x[0].astype(np.float64)
    assert np.all(np.signbit(d[d != 0]) == np.signbit(xs[d != 0]))
    for g in range(_groups(cols)):
        seg = slice(g * 128, min(cols, (g + 1) * 128))
        a = float(np.max(np.abs(xs[seg])))
        ac = max(a, FLOOR)
        sg = float(s[g, 0])
        top = float(np.max(np.abs(d[seg])))
        if mode == quant.MODE_MAXABS:
            if a >= FLOOR:
                assert top == 448.0
            else:
                assert top < 448.0 and sg == np.float32(FLOOR / 448.0)
        else:
            mant, _ = np.frexp(sg)
            assert mant == 0.5                                   # an integral power of two
            assert 224.0 < ac / sg <= 448.0
            assert top <= 448.0 and (a < FLOOR or top >= 224.0)
        # error bound: half an E4M3 step of the scaled magnitude, plus the
        # float32 roundings of the scale pair (zero in pow2 mode)
        y = np.abs(xs[seg]) / sg
        ulp = np.where(y >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(y, 2.0 ** -6))).astype(int) - 3),
                       2.0 ** -9)
        bound = sg * 0.5 * ulp * (1 + 2.0 ** -20) + 2.0 ** -21 * np.abs(xs[seg])
        assert np.all(np.abs(xs[seg] - d[seg] * sg) <= bound)


@SETTINGS
@given(rows=st.integers(1, 300), cols=st.integers(1, 300), seed=st.integers(0, 2 ** 32 - 1),
       e=st.integers(-140, 110))
def test_128x128_block_max_maps_to_448(rows, cols, seed, e):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, cols)) * 2.0 ** e).astype(np.float32)
    if not np.all(np.isfinite(w)):
        return
    q, s = quant.quant_128x128(w, quant.MODE_MAXABS)
    br, bc = -(-rows // 128), -(-cols // 128)
    assert q.shape == (rows, cols) and s.shape == (br, bc)
    d = np.abs(e4m3.decode(q))
    for i in range(br):
        for j in range(bc):
            blk = (slice(i * 128, (i + 1) * 128), slice(j * 128, (j + 1) * 128))
            a = float(np.max(np.abs(w[blk].astype(np.float64))))
            top = float(np.max(d[blk]))
            assert top == 448.0 if a >= FLOOR else top < 448.0
