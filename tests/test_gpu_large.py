"""Inputs beyond 2^31 elements / bytes: every address past the 32-bit range is
formed correctly.  The tensors are drawn on the GPU (seeded); the oracle
recomputes sampled rows and columns whose offsets lie beyond 2^31."""

import numpy as np
import pytest
import torch

from oracle import gemm as og, quant as oq
from tests.helpers import assert_bytes_equal, host, host_bf16_as_f64, require_gpu
from workloads import device_fp8_codes, device_normal_bf16

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _bf16_rows_to_f32(t):
    return oq.bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def test_quantizers_beyond_2g_elements():
    """36864 x 65536 BF16 (2.4e9 elements): 1x128 rows and 128x1 columns past element 2^31, from the
    single-tiling and the one-pass quantizers."""
    fp8q = require_gpu()
    rows, cols = 36864, 65536
    x = device_normal_bf16(301, (rows, cols))
    q, s = fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, fp8q.MAXABS)
    far_rows = np.array([32768, 32769, rows - 2, rows - 1])                  # row * cols >= 2^31
    q_ref, s_ref = oq.quant_1x128(_bf16_rows_to_f32(x[far_rows]), "maxabs")
    assert_bytes_equal(host(q[far_rows]), q_ref, "1x128 codes")
    assert_bytes_equal(host(s[:, far_rows]), s_ref, "1x128 scales")
    del q, s
    qt, st = fp8q.fp8_quant_tile(x, fp8q.TILE_128x1, fp8q.POW2)
    far_cols = np.array([58368, 65535])                                      # col * rows >= 2^31 in q_t
    qt_ref, st_ref = oq.quant_128x1(_bf16_rows_to_f32(x[:, far_cols]), "pow2")
    assert_bytes_equal(host(qt[far_cols]), qt_ref, "128x1 codes")
    assert_bytes_equal(host(st[:, far_cols]), st_ref, "128x1 scales")
    q, s, qt, st = fp8q.fp8_quant_tile_dual(x, fp8q.MAXABS)                 # both tilings in one pass
    q_ref, s_ref = oq.quant_1x128(_bf16_rows_to_f32(x[far_rows]), "maxabs")
    assert_bytes_equal(host(q[far_rows]), q_ref, "one-pass 1x128 codes")
    assert_bytes_equal(host(s[:, far_rows]), s_ref, "one-pass 1x128 scales")
    qt_ref, st_ref = oq.quant_128x1(_bf16_rows_to_f32(x[:, far_cols]), "maxabs")
    assert_bytes_equal(host(qt[far_cols]), qt_ref, "one-pass 128x1 codes")
    assert_bytes_equal(host(st[:, far_cols]), st_ref, "one-pass 128x1 scales")
    del x, q, s, qt, st
    torch.cuda.empty_cache()


def test_gemm_a_operand_beyond_2g_bytes():
    """Fprop with A of 139264 x 16384 codes (2.28e9 bytes): rows on both sides of byte 2^31."""
    fp8q = require_gpu()
    m, n, k = 139264, 256, 16384
    qa = device_fp8_codes(311, (m, k))
    qb = device_fp8_codes(312, (n, k))
    g = torch.Generator(device="cuda").manual_seed(313)
    sa = torch.exp2(torch.rand((k // 128, m), generator=g, device="cuda") * 8 - 12)
    sb = torch.exp2(torch.rand((n // 128, k // 128), generator=g, device="cuda") * 8 - 12)
    c = fp8q.fp8_gemm_blockscaled(fp8q.FPROP, qa, sa, qb, sb)
    sample = np.array([0, 131071, 131072, 131073, m - 2, m - 1])              # row 131072 starts at byte 2^31
    ref = og.gemm_ref(host(qa[sample]), host(sa[:, sample]), host(qb), host(sb), og.FPROP)
    got = host_bf16_as_f64(c[sample])
    assert og.rel_frobenius(got, og.round_bf16(ref)) <= TOL
    del qa, qb, sa, sb, c
    torch.cuda.empty_cache()


LD_MAX = (1 << 31) // 512 - 128          # the largest GEMM operand leading dimension the C ABI accepts (bytes)


def _rows_at_max_ld(seed, rows, k):
    """rows x k codes as a view with leading dimension LD_MAX; the rest of each row is NaN codes."""
    buf = torch.full((rows, LD_MAX), 0x7F, dtype=torch.uint8, device="cuda")
    buf[:, :k] = device_fp8_codes(seed, (rows, k))
    return buf[:, :k]


@pytest.mark.parametrize("kind,path", [("fprop", "promoted"), ("wgrad", "promoted"), ("dgrad", "pow2_ab"),
                                       ("wgrad", "pow2_a")])
def test_gemm_at_the_largest_leading_dimension(kind, path):
    """A and B rows 4,194,176 bytes apart, the most the ABI accepts (a 256-row tile then spans 2^31 - 2^15 bytes
    of 32-bit buffer offsets): every output against the oracle, and no NaN from the codes beyond K."""
    fp8q = require_gpu()
    kinds = {"fprop": fp8q.FPROP, "dgrad": fp8q.DGRAD, "wgrad": fp8q.WGRAD}
    m = n = 256
    k = 384
    a = _rows_at_max_ld(321, m, k)
    b = _rows_at_max_ld(322, n, k)
    assert a.stride(0) == b.stride(0) == LD_MAX
    rng = np.random.default_rng(323)
    def scales(shape, pow2):                # exponents in [-12, -4), integral where the MFMA applies the scale
        e = rng.uniform(-12, -4, size=shape)
        return torch.from_numpy(np.exp2(np.floor(e) if pow2 else e).astype(np.float32)).cuda()
    sa = scales((k // 128, m), path != "promoted")
    sb = scales((k // 128, n) if kind == "wgrad" else (n // 128, k // 128), path == "pow2_ab")
    if path == "promoted":
        c = fp8q.fp8_gemm_blockscaled(kinds[kind], a, sa, b, sb, out_dtype=torch.float32)
    else:
        mask = fp8q.POW2_AB if path == "pow2_ab" else fp8q.POW2_A
        c = fp8q.fp8_gemm_blockscaled_pow2(kinds[kind], a, sa, b, sb, out_dtype=torch.float32, pow2_operands=mask)
    ref = og.gemm_ref(host(a.contiguous()), host(sa), host(b.contiguous()), host(sb), kind)
    got = host(c).astype(np.float64)
    assert np.all(np.isfinite(got))
    assert og.rel_frobenius(got, og.round_output(ref, "f32")) <= 2e-4
    del a, b, c
    torch.cuda.empty_cache()


def test_grouped_at_the_largest_leading_dimension():
    fp8q = require_gpu()
    gmap = torch.tensor([1, 0], dtype=torch.int32, device="cuda")
    m, n, k, groups = 256, 512, 256, 2
    a = _rows_at_max_ld(331, m, k)
    qb = device_fp8_codes(332, (groups, n, k))
    rng = np.random.default_rng(333)
    sa = torch.from_numpy(np.exp2(rng.uniform(-12, -4, size=(k // 128, m))).astype(np.float32)).cuda()
    sb = torch.from_numpy(np.exp2(rng.uniform(-12, -4, size=(groups, n // 128, k // 128))).astype(np.float32)).cuda()
    c = fp8q.fp8_gemm_blockscaled_grouped(gmap, a, sa, qb, sb, out_dtype=torch.float32)
    ref = og.grouped_ref(host(a.contiguous()), host(sa), host(qb), host(sb), host(gmap))
    got = host(c).astype(np.float64)
    assert np.all(np.isfinite(got))
    assert og.rel_frobenius(got, og.round_output(ref, "f32")) <= 2e-4
    del a, c
    torch.cuda.empty_cache()
