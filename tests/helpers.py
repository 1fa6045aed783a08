"""Shared plumbing for the GPU tests: host <-> device copies and comparisons."""

import numpy as np
import torch


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X; none is visible"
    import precision_fp8_quant_amd as fp8q      # fails loudly if libfp8q.so is missing
    return fp8q


def dev_bf16(bits):
    """uint16 BF16 bit patterns (numpy) -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def host_bf16_as_f64(t):
    bits = host(t)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32:
        got_b, want_b = got.view(np.uint32), want.view(np.uint32)
    else:
        got_b, want_b = got, want
    bad = np.nonzero(got_b != want_b)
    if bad[0].size:
        idx = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} mismatches, first at {idx}: "
                             f"got {got[idx]!r} want {want[idx]!r}")
