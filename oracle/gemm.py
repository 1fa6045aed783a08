"""Block-scaled FP8 GEMM reference (TEST INFRASTRUCTURE ONLY -- never imported by the product path).

What the pages fix:
    * per-group scaling factors run along the inner dimension K of the GEMM
      and are multiplied in as the dequantization step -- dssusan.co.kr FP8
      excerpt, paragraph 3; "Deepseek - Not For everyone", paragraph 4;
    * partial MMA results are promoted to full FP32 accumulation at a fixed
      interval along K -- dssusan.co.kr FP8 excerpt, paragraph 3 (the interval's
      symbol is lost in extraction); youlimart.com FP8 excerpt, paragraph 2;
      "FP8 mixed precision - ...", section "FP32-аккумуляция";
    * Fprop, Dgrad and Wgrad all run in FP8 -- youlimart.com FP8 excerpt,
      paragraph 2; dssusan.co.kr FP8 excerpt, paragraph 3;
    * the GEMMs take FP8 inputs and write BF16 or FP32 -- youlimart.com FP8
      excerpt, paragraph 3.

Problem solved here (every operand K-contiguous, C = A . B^T):
    A codes QA[M][K] with 1x128 scales SA[K/128][M];
    B codes QB[N][K] with either 128x128 block scales SB[N/128][K/128]
      (Fprop, Dgrad: the weight operand) or 1-D scales SB[K/128][N]
      (Wgrad: both operands 128x1-quantized along the token axis);
    C[m][n] = sum_g SA[g][m] * sigmaB(g, n) * sum_{k in g} dec(QA[m][k]) * dec(QB[n][k]).

Reading of the promotion interval: one K-group of 128 (the scales change at
every group boundary, so the dequantization multiply has to happen there).

The reference is exact up to a final float64 summation: dec(q) * 2^9 is an
integer of magnitude <= 229376, so every per-group partial is an integer below
2^43 and is computed exactly (int64 for small problems, float64 BLAS per
group otherwise -- any summation order is exact below 2^53).
"""

import numpy as np

from . import e4m3

GROUP = 128
FPROP, DGRAD, WGRAD = "fprop", "dgrad", "wgrad"
_INT_SCALE = 2.0 ** 9          # dec(q) * 2^9 is an integer for every E4M3 code
_PAIR_SCALE = 2.0 ** -18       # undo the integer scaling of both operands


def _ints(q):
    """dec(q) * 2^9 as exact int64 (NaN codes rejected)."""
    q = np.asarray(q, dtype=np.uint8)
    if np.any((q & 0x7F) == 0x7F):
        raise ValueError("NaN code in a GEMM operand")
    return (e4m3.decode(q) * _INT_SCALE).astype(np.int64)


def _sigma_b(sb, kind, g, n_idx):
    """Scale of B for K-group g at output columns n_idx (float64)."""
    sb = np.asarray(sb, dtype=np.float64)
    if kind in (FPROP, DGRAD):
        return sb[n_idx // GROUP, g]
    if kind == WGRAD:
        return sb[g, n_idx]
    raise ValueError(f"unknown GEMM kind {kind!r}")


def group_partials(qa, qb, exact_int=False):
    """List of per-K-group partials P_g[m][n] = sum_{k in g} IA[m][k]*IB[n][k].

    With exact_int the products use int64 arithmetic; otherwise a float64
    matmul per group, which is exact because all values are integers < 2^53.
    """
    ia, ib = _ints(qa), _ints(qb)
    k = ia.shape[1]
    if ib.shape[1] != k:
        raise ValueError("A and B disagree on K")
    parts = []
    for g in range(-(-k // GROUP)):
        sl = slice(g * GROUP, min(k, (g + 1) * GROUP))
        if exact_int:
            parts.append(ia[:, sl] @ ib[:, sl].T)
        else:
            parts.append(ia[:, sl].astype(np.float64) @ ib[:, sl].astype(np.float64).T)
    return parts


def gemm_ref(qa, sa, qb, sb, kind=FPROP, exact_int=False):
    """Float64 C_ref[M][N] of the block-scaled GEMM (no output rounding)."""
    qa, qb = np.asarray(qa), np.asarray(qb)
    m, n = qa.shape[0], qb.shape[0]
    sa = np.asarray(sa, dtype=np.float64)
    cols = np.arange(n)
    c = np.zeros((m, n), dtype=np.float64)
    for g, p in enumerate(group_partials(qa, qb, exact_int)):
        scale = sa[g][:, None] * _sigma_b(sb, kind, g, cols)[None, :]
        c += scale * (np.asarray(p, dtype=np.float64) * _PAIR_SCALE)
    return c


def gemm_ref_entries(qa, sa, qb, sb, rows, cols, kind=FPROP):
    """C_ref at the listed (rows[i], cols[i]) positions only (float64).

    Used for full-size problems where the whole product is too costly on the
    CPU: each sampled entry is computed exactly per K-group in int64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ia = _ints(np.asarray(qa)[rows])            # [S][K]
    ib = _ints(np.asarray(qb)[cols])            # [S][K]
    k = ia.shape[1]
    sa = np.asarray(sa, dtype=np.float64)
    out = np.zeros(rows.shape[0], dtype=np.float64)
    for g in range(-(-k // GROUP)):
        sl = slice(g * GROUP, min(k, (g + 1) * GROUP))
        p = np.sum(ia[:, sl] * ib[:, sl], axis=1)                 # exact int64
        out += sa[g][rows] * _sigma_b(sb, kind, g, cols) * (p.astype(np.float64) * _PAIR_SCALE)
    return out


def grouped_ref(qa, sa, qb, sb, group_of_mtile):
    """Grouped (MoE) Fprop: rows of each 128-row M tile use that tile's group.

    qa [M_total][K], sa [K/128][M_total], qb [G][N][K], sb [G][N/128][K/128],
    group_of_mtile [M_total/128]. Returns float64 C_ref[M_total][N].
    """
    qa = np.asarray(qa)
    gmap = np.asarray(group_of_mtile, dtype=np.int64)
    m_total = qa.shape[0]
    n = np.asarray(qb).shape[1]
    sa = np.asarray(sa)
    c = np.zeros((m_total, n), dtype=np.float64)
    for t, grp in enumerate(gmap):
        rs = slice(t * GROUP, (t + 1) * GROUP)
        c[rs] = gemm_ref(qa[rs], sa[:, rs], qb[grp], sb[grp], FPROP)
    return c


def round_bf16(x):
    """Round float64 values to the nearest BF16 (ties to even), returned as float64.

    Single rounding straight from float64 (no float32 detour): keep 8
    significant bits, with the quantum floored at the BF16 subnormal step 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                                # |x| in [2^(e-1), 2^e)
    q = np.maximum(e.astype(np.int64) - 8, -133)      # exponent of one BF16 ulp
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)      # rint rounds half to even


def bf16_bits(x):
    """BF16 bit patterns (uint16) of float64 values already on the BF16 grid."""
    f = np.asarray(x, dtype=np.float32)               # exact for BF16 values
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_output(c_ref, out_dtype):
    """The output a kernel should aim for: C_ref rounded once to its dtype."""
    if out_dtype == "f32":
        return np.asarray(c_ref, dtype=np.float64).astype(np.float32).astype(np.float64)
    if out_dtype == "bf16":
        return round_bf16(c_ref)
    raise ValueError(f"unknown output dtype {out_dtype!r}")


def rel_frobenius(c, ref):
    """||c - ref||_F / ||ref||_F in float64."""
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(c - ref)
    return float(num / den) if den > 0 else float(num)
