"""Stream semantics of the C ABI: all work is enqueued on the caller's stream
(never the default one behind its back) and nothing synchronises, so the
path runs on user streams and can be captured into a HIP graph and
replayed."""

import numpy as np
import pytest
import torch

from tests.helpers import dev_bf16, host, require_gpu
from workloads import add_outliers, normal_f32, to_bf16_bits

pytestmark = pytest.mark.gpu


def _inputs(seed, m=512, n=768, k=1024):
    rng = np.random.default_rng(seed)
    x = dev_bf16(to_bf16_bits(add_outliers(rng, normal_f32(rng, (m, k), 1.0), 0.005, 50.0)))
    w = dev_bf16(to_bf16_bits(normal_f32(rng, (n, k), 0.02)))
    return x, w


def _fprop(fp8q, x, w, stream=None):
    qx, sx = fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, fp8q.MAXABS, stream=stream)
    qw, sw = fp8q.fp8_quant_block(w, fp8q.MAXABS, stream=stream)
    return fp8q.fp8_gemm_blockscaled(fp8q.FPROP, qx, sx, qw, sw, stream=stream)


def test_pipeline_on_a_user_stream_while_the_default_stream_is_busy():
    fp8q = require_gpu()
    x, w = _inputs(501)
    want = host(_fprop(fp8q, x, w))
    busy = torch.randn(4096, 4096, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(4):                               # keep the default stream busy meanwhile
        busy = busy @ busy.t() * 1e-3
    with torch.cuda.stream(s):
        got = _fprop(fp8q, x, w, stream=s)            # explicit stream argument
    s.synchronize()
    assert np.array_equal(host(got), want)


def test_work_is_ordered_on_the_callers_stream():
    """A torch write on stream s followed by a quantization on s sees the write."""
    fp8q = require_gpu()
    s = torch.cuda.Stream()
    x = torch.zeros(256, 512, device="cuda", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        x.fill_(3.0)
        q, sc = fp8q.fp8_quant_tile(x, fp8q.TILE_1x128, fp8q.POW2)    # current stream = s
    s.synchronize()
    assert torch.all(sc == 2.0 ** -7).item()          # 3 / 448 -> pow2 scale 2^-7
    assert torch.all(q == 0x7C).item()                # 3 * 2^7 = 384 = 1.5 * 2^8 = E4M3 0x7C


def test_pipeline_captured_in_a_hip_graph_and_replayed():
    """Quantize X and W and run Fprop inside a captured graph; between replays new
    inputs are copied into the captured buffers (eager work and synchronisation in
    between), and every replay must equal the eager result bit for bit."""
    fp8q = require_gpu()
    x_buf, w_buf = _inputs(511)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                        # warm-up outside capture
        _fprop(fp8q, x_buf, w_buf)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_buf = _fprop(fp8q, x_buf, w_buf)
    torch.cuda.synchronize()
    for seed in (521, 522, 523, 524):
        x, w = _inputs(seed)
        want = host(_fprop(fp8q, x, w))               # eager, on the default stream
        x_buf.copy_(x)
        w_buf.copy_(w)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y_buf), want), seed


def test_ksplit_last_wave_captured_in_a_hip_graph_and_replayed():
    """The same for a GEMM whose half-full last wave runs as K halves (M=512, N=129*256, K=384, BF16 out): the
    split grid, the kernel adding the halves (both through scratch in C) and the head grid replay in order, and
    every replay equals the eager result bit for bit."""
    fp8q = require_gpu()
    shape = dict(m=512, n=129 * 256, k=384)
    x_buf, w_buf = _inputs(611, **shape)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _fprop(fp8q, x_buf, w_buf)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_buf = _fprop(fp8q, x_buf, w_buf)
    torch.cuda.synchronize()
    for seed in (621, 622, 623):
        x, w = _inputs(seed, **shape)
        want = host(_fprop(fp8q, x, w))
        x_buf.copy_(x)
        w_buf.copy_(w)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y_buf), want), seed
