"""The C ABI from plain C: tests/c_client/fp8q_client.c includes include/fp8q.h,
links libfp8q.so and calls the entry points directly (no Python in between).
Its validation mode runs without a GPU; its run mode quantizes X and W and
multiplies them on the GPU, and its outputs are checked against the oracle."""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import gemm as og, quant as oq
from tests.helpers import assert_bytes_equal
from workloads import add_outliers, normal_f32, to_bf16_bits

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "precision_fp8_quant_amd")
SRC = os.path.join(ROOT, "tests", "c_client", "fp8q_client.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="session")
def client(tmp_path_factory):
    if not os.path.exists(os.path.join(LIB_DIR, "libfp8q.so")):
        pytest.skip("libfp8q.so not built")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("c_client") / "fp8q_client")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{ROOT}/include", SRC, f"-L{LIB_DIR}", "-lfp8q", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{LIB_DIR}", f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_client_validation(client):
    res = subprocess.run([client, "check"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    assert "validation ok" in res.stdout


@pytest.mark.gpu
def test_c_client_quantize_and_fprop(client, tmp_path):
    m, n, k = 256, 384, 512
    rng = np.random.default_rng(97)
    x = to_bf16_bits(add_outliers(rng, normal_f32(rng, (m, k), 1.0), 0.005, 50.0))
    w = to_bf16_bits(normal_f32(rng, (n, k), 0.02))
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as fh:
        np.array([m, n, k], np.int64).tofile(fh)
        x.tofile(fh)
        w.tofile(fh)
    res = subprocess.run([client, "run", str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    buf = open(out, "rb").read()
    sizes = [("qx", m * k, np.uint8), ("sx", (k // 128) * m, np.float32), ("qw", n * k, np.uint8),
             ("sw", (n // 128) * (k // 128), np.float32), ("y", m * n, np.uint16)]
    got, off = {}, 0
    for name, count, dt in sizes:
        nbytes = count * np.dtype(dt).itemsize
        got[name] = np.frombuffer(buf[off:off + nbytes], dtype=dt)
        off += nbytes
    assert off == len(buf)
    qx, sx = oq.quant_1x128(oq.bf16_bits_to_f32(x), "maxabs")
    qw, sw = oq.quant_128x128(oq.bf16_bits_to_f32(w), "maxabs")
    assert_bytes_equal(got["qx"].reshape(m, k), qx, "codes of X")
    assert_bytes_equal(got["sx"].reshape(k // 128, m), sx, "scales of X")
    assert_bytes_equal(got["qw"].reshape(n, k), qw, "codes of W")
    assert_bytes_equal(got["sw"].reshape(n // 128, k // 128), sw, "scales of W")
    y = (got["y"].astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64).reshape(m, n)
    ref = og.gemm_ref(qx, sx, qw, sw, og.FPROP)
    assert og.rel_frobenius(y, og.round_bf16(ref)) <= 1e-3
