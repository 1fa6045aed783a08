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
