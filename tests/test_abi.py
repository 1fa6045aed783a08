"""The C-ABI library loads, exports every entry point declared in include/fp8q.h,
and rejects bad arguments before anything is launched (CPU only: no call here
reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")

fp8q = pytest.importorskip("precision_fp8_quant_amd", reason="libfp8q.so not built")

A = 0x10000          # fake, 16-byte aligned "device" addresses: never dereferenced,
B = 0x20000000       # because every call below fails validation first
C = 0x40000000
D = 0x60000000


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert names == {"fp8_quant_tile", "fp8_quant_tile_dual", "fp8_quant_block", "fp8_gemm_blockscaled",
                     "fp8_gemm_blockscaled_grouped", "fp8_requant_1x128_to_128x1",
                     "fp8_gemm_blockscaled_pow2", "fp8q_status_string",
                     "fp8q_abi_version"}
    raw = ctypes.CDLL(fp8q.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(fp8q.SIGNATURES) == names


def test_version_and_status_strings():
    assert fp8q.lib.fp8q_abi_version() == 104
    for s in range(8):
        assert fp8q.status_string(s).startswith("FP8Q_")
    assert fp8q.status_string(99) == "unknown fp8q status"


def _tile(**kw):
    args = dict(x=A, dt=fp8q.BF16, rows=128, cols=256, ldx=256, tile=fp8q.TILE_1x128, mode=fp8q.MAXABS,
                q=B, ldq=256, s=C)
    args.update(kw)
    return fp8q.lib.fp8_quant_tile(args["x"], args["dt"], args["rows"], args["cols"], args["ldx"], args["tile"],
                                   args["mode"], args["q"], args["ldq"], args["s"], None)


def test_quant_tile_validation():
    assert _tile(rows=0) == fp8q.OK and _tile(cols=0, x=None) == fp8q.OK   # empty: no-op
    assert _tile(dt=7) == fp8q.ERR_ARG
    assert _tile(tile=5) == fp8q.ERR_ARG
    assert _tile(mode=2) == fp8q.ERR_ARG
    assert _tile(rows=-1) == fp8q.ERR_SHAPE
    assert _tile(x=None) == fp8q.ERR_NULL
    assert _tile(s=None) == fp8q.ERR_NULL
    assert _tile(ldx=128) == fp8q.ERR_SHAPE
    assert _tile(x=A + 2) == fp8q.ERR_ALIGN
    assert _tile(ldx=260) == fp8q.ERR_ALIGN          # 520 bytes is not a multiple of 16
    assert _tile(cols=200, ldx=200, ldq=208) == fp8q.ERR_UNSUPPORTED
    assert _tile(tile=fp8q.TILE_128x1, rows=100, ldq=256) == fp8q.ERR_UNSUPPORTED
    assert _tile(tile=fp8q.TILE_128x1, cols=252, ldx=256, ldq=128) == fp8q.ERR_UNSUPPORTED
    assert _tile(q=A + 64) == fp8q.ERR_ALIAS         # codes overlap the input
    assert _tile(s=B + 1024) == fp8q.ERR_ALIAS       # scales overlap the codes


def _block(**kw):
    args = dict(w=A, dt=fp8q.F32, rows=256, cols=384, ldw=384, mode=fp8q.POW2, q=B, ldq=384, s=C,
                qt=None, ldqt=0, st=None)
    args.update(kw)
    return fp8q.lib.fp8_quant_block(args["w"], args["dt"], args["rows"], args["cols"], args["ldw"], args["mode"],
                                    args["q"], args["ldq"], args["s"], args["qt"], args["ldqt"], args["st"],
                                    None)


def test_quant_block_validation():
    assert _block(rows=0, w=None) == fp8q.OK
    assert _block(mode=9) == fp8q.ERR_ARG
    assert _block(q=None) == fp8q.ERR_NULL
    assert _block(qt=D, ldqt=256) == fp8q.ERR_NULL             # q_t without scales_t
    assert _block(st=D) == fp8q.ERR_ARG                         # scales_t without q_t
    assert _block(qt=D, ldqt=128, st=D + 0x100000) == fp8q.ERR_SHAPE
    assert _block(rows=200) == fp8q.ERR_UNSUPPORTED
    assert _block(ldq=392) == fp8q.ERR_ALIGN
    assert _block(qt=B + 16, ldqt=256, st=D) == fp8q.ERR_ALIAS  # transposed codes overlap codes


def _dual(**kw):
    args = dict(x=A, dt=fp8q.BF16, rows=256, cols=384, ldx=384, mode=fp8q.MAXABS, q=B, ldq=384, s=C,
                qt=D, ldqt=256, st=0x70000000)
    args.update(kw)
    return fp8q.lib.fp8_quant_tile_dual(args["x"], args["dt"], args["rows"], args["cols"], args["ldx"],
                                        args["mode"], args["q"], args["ldq"], args["s"], args["qt"], args["ldqt"],
                                        args["st"], None)


def test_quant_tile_dual_validation():
    assert _dual(rows=0, x=None) == fp8q.OK and _dual(cols=0, q=None) == fp8q.OK   # empty: no-op
    assert _dual(dt=3) == fp8q.ERR_ARG
    assert _dual(mode=2) == fp8q.ERR_ARG
    assert _dual(cols=-128) == fp8q.ERR_SHAPE
    for name in ("x", "q", "s", "qt", "st"):                    # all four outputs are required
        assert _dual(**{name: None}) == fp8q.ERR_NULL, name
    assert _dual(ldx=256) == fp8q.ERR_SHAPE
    assert _dual(ldq=256) == fp8q.ERR_SHAPE
    assert _dual(ldqt=128) == fp8q.ERR_SHAPE
    assert _dual(st=0x70000004) == fp8q.ERR_ALIGN
    assert _dual(ldqt=264) == fp8q.ERR_ALIGN
    assert _dual(rows=200, ldqt=208) == fp8q.ERR_UNSUPPORTED    # rows must be whole 128-row tiles
    assert _dual(cols=264, ldx=264, ldq=272) == fp8q.ERR_UNSUPPORTED
    assert _dual(qt=B + 4096) == fp8q.ERR_ALIAS                 # transposed codes overlap the 1x128 codes
    assert _dual(st=C + 16) == fp8q.ERR_ALIAS                   # the two scale arrays overlap
    assert _dual(q=A + 256) == fp8q.ERR_ALIAS                   # codes overlap the input


def _gemm(fn="fp8_gemm_blockscaled", **kw):
    args = dict(kind=fp8q.FPROP, M=256, N=256, K=512, a=A, lda=512, sa=B, b=C, ldb=512, sb=D,
                c=0x7000000, cdt=fp8q.BF16, ldc=256, acc=0, pow2=fp8q.POW2_AB)
    args.update(kw)
    extra = (args["pow2"],) if fn == "fp8_gemm_blockscaled_pow2" else ()
    return getattr(fp8q.lib, fn)(args["kind"], args["M"], args["N"], args["K"], args["a"], args["lda"],
                                 args["sa"], args["b"], args["ldb"], args["sb"], args["c"], args["cdt"],
                                 args["ldc"], args["acc"], *extra, None)


@pytest.mark.parametrize("fn", ["fp8_gemm_blockscaled", "fp8_gemm_blockscaled_pow2"])
def test_gemm_validation(fn):
    assert _gemm(fn, M=0) == fp8q.OK
    assert _gemm(fn, kind=3) == fp8q.ERR_ARG
    assert _gemm(fn, cdt=4) == fp8q.ERR_ARG
    assert _gemm(fn, acc=2) == fp8q.ERR_ARG
    assert _gemm(fn, K=-128) == fp8q.ERR_SHAPE
    assert _gemm(fn, c=None) == fp8q.ERR_NULL
    assert _gemm(fn, sb=None) == fp8q.ERR_NULL
    assert _gemm(fn, lda=256) == fp8q.ERR_SHAPE
    assert _gemm(fn, ldc=200) == fp8q.ERR_SHAPE
    assert _gemm(fn, b=C + 8) == fp8q.ERR_ALIGN
    assert _gemm(fn, M=200) == fp8q.ERR_UNSUPPORTED
    assert _gemm(fn, acc=1) == fp8q.ERR_UNSUPPORTED              # accumulate needs FP32 output
    assert _gemm(fn, lda=1 << 22) == fp8q.ERR_UNSUPPORTED         # rows of 4 MiB: beyond 32-bit tile offsets
    assert _gemm(fn, ldb=(1 << 22) - 112) == fp8q.ERR_UNSUPPORTED      # just above 4,194,176
    assert _gemm(fn, c=A + 4096) == fp8q.ERR_ALIAS


def test_pow2_gemm_operand_mask_validation():
    for bad in (0, 4, -1):
        assert _gemm("fp8_gemm_blockscaled_pow2", pow2=bad) == fp8q.ERR_ARG
    for ok in (fp8q.POW2_A, fp8q.POW2_B, fp8q.POW2_AB):
        assert _gemm("fp8_gemm_blockscaled_pow2", pow2=ok, M=0) == fp8q.OK


def _grouped(**kw):
    args = dict(G=4, M=512, N=256, K=256, gmap=0x9000000, a=A, lda=256, sa=B, b=C, sb=D, c=0x7000000,
                cdt=fp8q.BF16, ldc=256)
    args.update(kw)
    return fp8q.lib.fp8_gemm_blockscaled_grouped(args["G"], args["M"], args["N"], args["K"], args["gmap"], args["a"],
                                                 args["lda"], args["sa"], args["b"], args["sb"], args["c"],
                                                 args["cdt"], args["ldc"], None)


def test_grouped_validation():
    assert _grouped(M=0) == fp8q.OK
    assert _grouped(G=0) == fp8q.ERR_SHAPE
    assert _grouped(gmap=None) == fp8q.ERR_NULL
    assert _grouped(gmap=0x9000002) == fp8q.ERR_ALIGN
    assert _grouped(N=192) == fp8q.ERR_UNSUPPORTED
    assert _grouped(c=C + 0x100) == fp8q.ERR_ALIAS


def test_binding_raises_on_error_status():
    with pytest.raises(fp8q.Fp8qError):
        fp8q._check(fp8q.ERR_SHAPE)


def _requant(**kw):
    args = dict(q=A, rows=256, cols=384, ldq=384, s=B, mode=fp8q.POW2, qt=C, ldqt=256, st=D)
    args.update(kw)
    return fp8q.lib.fp8_requant_1x128_to_128x1(args["q"], args["rows"], args["cols"], args["ldq"], args["s"],
                                               args["mode"], args["qt"], args["ldqt"], args["st"], None)


def test_requant_validation():
    assert _requant(rows=0, q=None) == fp8q.OK
    assert _requant(mode=3) == fp8q.ERR_ARG
    assert _requant(cols=-128) == fp8q.ERR_SHAPE
    for k in ("q", "s", "qt", "st"):
        assert _requant(**{k: None}) == fp8q.ERR_NULL
    assert _requant(ldq=256) == fp8q.ERR_SHAPE
    assert _requant(ldqt=128) == fp8q.ERR_SHAPE
    assert _requant(q=A + 8) == fp8q.ERR_ALIGN
    assert _requant(ldq=392) == fp8q.ERR_ALIGN
    assert _requant(rows=200, ldqt=208) == fp8q.ERR_UNSUPPORTED
    assert _requant(cols=200, ldq=208) == fp8q.ERR_UNSUPPORTED
    assert _requant(qt=A + 256) == fp8q.ERR_ALIAS          # codes out over codes in
    assert _requant(st=C + 1024) == fp8q.ERR_ALIAS         # scales out inside codes out
    assert _requant(st=B) == fp8q.ERR_ALIAS                # scales out over scales in


def test_import_fails_loudly_without_the_library(tmp_path):
    """The binding has no CPU fallback: a package directory without libfp8q.so
    refuses to import, naming the missing library."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "precision_fp8_quant_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "precision_fp8_quant_amd", "__init__.py"), pkg / "__init__.py")
    res = subprocess.run([sys.executable, "-c", "import precision_fp8_quant_amd"], cwd=tmp_path,
                         env={**os.environ, "PYTHONPATH": str(tmp_path)}, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0
    assert "libfp8q.so is missing" in res.stderr and "no CPU fallback" in res.stderr
