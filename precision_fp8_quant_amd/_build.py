"""Compile the fp8q HIP library (libfp8q.so) in-tree for gfx950.

Every kernel is hand-written HIP for CDNA4; this only drives hipcc.  The
library is linked into ``precision_fp8_quant_amd/libfp8q.so`` next to the
binding, so it travels with the source tree.
"""

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfp8q.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

DEVICE_SOURCES = ["quant.hip", "gemm.hip", "gemm_pow2.hip"]
HOST_SOURCES = ["abi.cpp"]

# -ffp-contract=off: the quantizer's scale-multiply-then-round sequence must be
# exactly the stated FP32 operations (no fused multiply-add formed behind our
# back); the GEMM asks for its FMAs explicitly.
# -packed-fp32-ops off: keep the compiler from forming packed FP32 VALU ops.
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-I", INCLUDE, "-I", CSRC]
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument"]
# -amdgpu-mfma-vgpr-form: MFMA results go straight to VGPRs, where the FP32
# promotion FMAs read them (no v_accvgpr_read copies).  Not for the
# hardware-scaled GEMM, whose accumulators stay in AGPRs inside the MFMA chain.
PER_SOURCE_FLAGS = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def build(verbose=False, extra_flags=()):
    """Compile every source and link libfp8q.so (always recompiles)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append([HIPCC, *COMMON_FLAGS, *DEVICE_FLAGS, *PER_SOURCE_FLAGS.get(src, []), *extra_flags,
                     "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append([HIPCC, *COMMON_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


TEST_PROBE_SRC = os.path.join(os.path.dirname(PKG_DIR), "tests", "hip", "scale_div_probe.hip")
TEST_PROBE_LIB = os.path.join(os.path.dirname(PKG_DIR), "tests", "hip", "libfp8q_divprobe.so")


def build_test_probe(verbose=False):
    """Compile the GPU test helper tests/hip/scale_div_probe.hip (not part of libfp8q.so) with the library's
    device flags, so that it exercises the same code as the quantizers."""
    tmp = TEST_PROBE_LIB + ".tmp"
    _run([HIPCC, *COMMON_FLAGS, *DEVICE_FLAGS, "-shared", TEST_PROBE_SRC, "-o", tmp], verbose)
    os.replace(tmp, TEST_PROBE_LIB)
    return TEST_PROBE_LIB


if __name__ == "__main__":
    print(build(verbose=True))
