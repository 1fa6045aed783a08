"""The quantizers' scale divisions on the GPU against IEEE division, for every input.

The max-abs scale pair is s = fl32(a / 448) and inv = fl32(448 / a) for the
group max-abs a >= 448 * 2^-126 (the floor the quantizers apply), a single
correctly-rounded float32 division each.  On the GPU both come from a
reciprocal estimate plus one FMA correction (fp8q_device.h).  This test runs
those device functions, built with the library's flags into a small test
helper (tests/hip/scale_div_probe.hip), over all 2,057,306,112 float32 values
in [448 * 2^-126, FLT_MAX] and compares every result bit for bit with numpy's
float32 division, which is IEEE round-to-nearest-even.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

from tests.helpers import require_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tests", "hip", "libfp8q_divprobe.so")

FIRST = 0x04E00000          # 448 * 2^-126
LAST = 0x7F7FFFFF           # FLT_MAX
CHUNK = 1 << 27


@pytest.mark.gpu
def test_scale_divisions_match_ieee_for_every_float32_in_range():
    require_gpu()
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE)
    lib.fp8q_scale_div_probe.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.fp8q_scale_div_probe.restype = ctypes.c_int
    s_dev = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    inv_dev = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    f448 = np.float32(448.0)
    total = 0
    first = FIRST
    while first <= LAST:
        n = min(CHUNK, LAST - first + 1)
        assert lib.fp8q_scale_div_probe(first, n, s_dev.data_ptr(), inv_dev.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        a = np.arange(first, first + n, dtype=np.uint32).view(np.float32)      # first + n <= 2^31
        s_gpu = s_dev[:n].cpu().numpy().view(np.uint32)
        inv_gpu = inv_dev[:n].cpu().numpy().view(np.uint32)
        s_ref = (a / f448).view(np.uint32)
        inv_ref = (f448 / a).view(np.uint32)
        bad_s = np.flatnonzero(s_gpu != s_ref)
        bad_i = np.flatnonzero(inv_gpu != inv_ref)
        assert bad_s.size == 0, f"a/448: {bad_s.size} mismatches, first at bits {first + int(bad_s[0]):#010x}"
        assert bad_i.size == 0, f"448/a: {bad_i.size} mismatches, first at bits {first + int(bad_i[0]):#010x}"
        total += n
        first += n
    assert total == LAST - FIRST + 1 == 2_057_306_112
