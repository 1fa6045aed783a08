"""The C ABI's argument validation built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer and driven with adversarial sizes (CPU only).

abi.cpp is compiled with g++ together with host stand-ins for the HIP
launchers (tests/c_client/stub_launch.cpp), so no GPU and no HIP runtime are
needed; tests/c_client/abi_adversarial.c calls every entry point with sizes
whose byte extents overflow, buffers that wrap past the top of the address
space and tile counts beyond one grid.  Any signed overflow, out-of-bounds
access or other undefined behaviour in the validation aborts the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "precision_fp8_quant_amd", "csrc")
CLIENT = os.path.join(ROOT, "tests", "c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.fixture(scope="module")
def adversarial_exe(tmp_path_factory):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if gxx is None or gcc is None:
        pytest.skip("no host compiler")
    d = tmp_path_factory.mktemp("abi_san")
    inc = [f"-I{ROOT}/include", f"-I{CSRC}", f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src, cc, std in ((os.path.join(CSRC, "abi.cpp"), gxx, "-std=c++17"),
                         (os.path.join(CLIENT, "stub_launch.cpp"), gxx, "-std=c++17"),
                         (os.path.join(CLIENT, "abi_adversarial.c"), gcc, "-std=c11")):
        obj = str(d / (os.path.basename(src) + ".o"))
        subprocess.run([cc, std, "-Wall", "-Werror", *SAN, *inc, "-c", src, "-o", obj],
                       check=True, capture_output=True, text=True)
        objs.append(obj)
    exe = str(d / "abi_adversarial")
    subprocess.run([gxx, *SAN, *objs, "-o", exe], check=True, capture_output=True, text=True)
    return exe


def test_validation_under_sanitizers(adversarial_exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([adversarial_exe], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "adversarial validation ok (3 launches reached)" in res.stdout
    assert "runtime error" not in res.stderr and "ERROR: AddressSanitizer" not in res.stderr
