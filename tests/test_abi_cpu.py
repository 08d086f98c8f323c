"""The C-ABI library loads, exports every function include/scaled_fp8.h declares, reports a
missing device, and rejects bad arguments before launching anything (CPU only)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scaled_fp8.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|char\s*\*|const char\s*\*)\s*(fp8_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    assert names == sorted(["fp8_device_check", "fp8_recipe_update", "fp8_quantize", "fp8_quantize_diag",
                            "fp8_cast_transpose", "fp8_cast_transpose_blockwise", "fp8_gemm", "fp8_gemm_fused",
                            "fp8_layernorm_quantize", "fp8_last_error"])


def test_library_exports_every_declared_symbol():
    import scaled_quantize_gemm_amd as sq

    lib = ctypes.CDLL(sq.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(sq.EXPORTED) == set(_declared())


def test_header_constants_match_binding():
    import scaled_quantize_gemm_amd as sq

    src = open(HEADER).read()
    for name in ["FP8_E4M3", "FP8_E5M2", "HP_F32", "HP_BF16", "OUT_F32", "OUT_BF16", "OUT_E4M3", "OUT_E5M2",
                 "FP8_ACT_NONE", "FP8_ACT_GELU", "FP8_ACT_SWIGLU", "FP8_SCALE_TENSOR",
                 "FP8_SCALE_TILE_1x128", "FP8_SCALE_BLOCK_128x128", "FP8_SCALE_MX_1x32", "FP8_OK", "FP8_ERR_ARG",
                 "FP8_ERR_SHAPE", "FP8_ERR_DTYPE", "FP8_ERR_DEVICE", "FP8_ERR_LAUNCH"]:
        m = re.search(rf"\b{name}\s*=\s*(-?\d+)", src)
        assert m, name
        assert int(m.group(1)) == getattr(sq, name), name


def _no_gpu():
    import torch

    return not torch.cuda.is_available()


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device path")
def test_device_check_without_gpu_reports_error():
    import scaled_quantize_gemm_amd as sq

    ok, why = sq.fp8_device_check(0)
    assert not ok and why
    assert sq.fp8_last_error()


def test_argument_errors_return_before_launch():
    """Invalid arguments are rejected on the host with the documented codes (no kernel runs)."""
    import scaled_quantize_gemm_amd as sq

    lib = sq.lib
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first
    # quantize: bad dtype, bad fmt, bad granularity, TILE with ragged cols, MX ragged cols, negative shape
    assert lib.fp8_quantize(fake, 7, 4, 128, 0, 0, fake, None, fake, None, None) == sq.FP8_ERR_DTYPE
    assert lib.fp8_quantize(fake, 1, 4, 128, 5, 0, fake, None, fake, None, None) == sq.FP8_ERR_ARG
    assert lib.fp8_quantize(fake, 1, 4, 128, 0, 9, fake, None, fake, None, None) == sq.FP8_ERR_ARG
    assert lib.fp8_quantize(fake, 1, 4, 100, 0, 1, None, None, fake, fake, None) == sq.FP8_ERR_SHAPE
    assert lib.fp8_quantize(fake, 1, 4, 48, 0, 3, None, None, fake, fake, None) == sq.FP8_ERR_SHAPE
    assert lib.fp8_quantize(fake, 1, -1, 128, 0, 0, fake, None, fake, None, None) == sq.FP8_ERR_SHAPE
    assert lib.fp8_quantize(fake, 1, 4, 128, 0, 0, None, None, fake, None, None) == sq.FP8_ERR_ARG  # no scale
    assert lib.fp8_quantize(fake, 1, 4, 128, 0, 1, fake, None, fake, fake, None) == sq.FP8_ERR_ARG  # scale w/ TILE
    misaligned = ctypes.c_void_p(0x100008)
    assert lib.fp8_quantize(misaligned, 1, 4, 128, 0, 0, fake, None, fake, None, None) == sq.FP8_ERR_ARG
    assert "aligned" in sq.fp8_last_error()
    # empty input is valid and enqueues nothing
    assert lib.fp8_quantize(None, 1, 0, 128, 0, 0, fake, None, None, None, None) == sq.FP8_OK
    # cast-transpose
    assert lib.fp8_cast_transpose(fake, 1, 4, 4, 0, None, None, fake, fake, None) == sq.FP8_ERR_ARG
    assert lib.fp8_cast_transpose(fake, 2, 4, 4, 0, fake, None, fake, fake, None) == sq.FP8_ERR_DTYPE
    assert lib.fp8_cast_transpose(None, 1, 0, 5, 0, fake, None, None, None, None) == sq.FP8_OK
    # quantize with diagnostics: counts required and 8-byte aligned
    qd = lib.fp8_quantize_diag
    assert qd(fake, 1, 4, 128, 0, fake, None, fake, None, None) == sq.FP8_ERR_ARG
    assert qd(fake, 1, 4, 128, 0, fake, None, fake, ctypes.c_void_p(0x100004), None) == sq.FP8_ERR_ARG
    assert qd(fake, 3, 4, 128, 0, fake, None, fake, fake, None) == sq.FP8_ERR_DTYPE
    assert qd(None, 1, 0, 128, 0, fake, None, None, fake, None) == sq.FP8_OK
    # blockwise cast-transpose: granularity, shapes that are not multiples of 128, dtype, empty
    ct = lib.fp8_cast_transpose_blockwise
    assert ct(fake, 1, 128, 128, 0, 0, fake, fake, fake, fake, None) == sq.FP8_ERR_ARG
    assert ct(fake, 1, 128, 128, 0, 3, fake, fake, fake, fake, None) == sq.FP8_ERR_ARG
    assert ct(fake, 1, 100, 128, 0, 1, fake, fake, fake, fake, None) == sq.FP8_ERR_SHAPE
    assert ct(fake, 1, 128, 200, 0, 2, fake, fake, fake, fake, None) == sq.FP8_ERR_SHAPE
    assert ct(fake, 5, 128, 128, 0, 1, fake, fake, fake, fake, None) == sq.FP8_ERR_DTYPE
    assert ct(fake, 1, 128, 128, 0, 1, fake, None, fake, fake, None) == sq.FP8_ERR_ARG
    assert ct(None, 1, 0, 128, 0, 2, None, None, None, None, None) == sq.FP8_OK
    # gemm: K not a multiple of 128, bad pair, bad out dtype, empty
    assert lib.fp8_gemm(fake, 0, fake, 0, fake, 0, fake, 0, fake, 0, 4, 4, 100, None) == sq.FP8_ERR_SHAPE
    assert lib.fp8_gemm(fake, 0, fake, 0, fake, 0, fake, 3, fake, 0, 4, 4, 128, None) == sq.FP8_ERR_ARG
    assert "granularity" in sq.fp8_last_error()
    assert lib.fp8_gemm(fake, 0, fake, 2, fake, 0, fake, 1, fake, 0, 4, 4, 128, None) == sq.FP8_ERR_ARG
    assert lib.fp8_gemm(fake, 0, fake, 1, fake, 0, fake, 3, fake, 0, 4, 4, 128, None) == sq.FP8_ERR_ARG
    assert lib.fp8_gemm(fake, 0, fake, 0, fake, 0, fake, 0, fake, 7, 4, 4, 128, None) == sq.FP8_ERR_DTYPE
    assert lib.fp8_gemm(fake, 0, fake, 0, fake, 0, fake, 0, fake, 0, 0, 4, 128, None) == sq.FP8_OK
    assert lib.fp8_gemm(fake, 2, fake, 0, fake, 0, fake, 0, fake, 0, 4, 4, 128, None) == sq.FP8_ERR_ARG
    # fused gemm: bad act, SwiGLU with odd N, FP8 output without scale / amax, bad out and bias
    # dtypes, C not 16-byte aligned, bad granularity pair, empty
    fg = lib.fp8_gemm_fused
    assert fg(fake, 0, fake, 0, fake, 0, fake, 0, None, 0, 9, None, fake, 0, None, None, 4, 4, 128, None) == sq.FP8_ERR_ARG
    assert fg(fake, 0, fake, 0, fake, 0, fake, 0, None, 0, 2, None, fake, 0, None, None, 4, 5, 128, None) == sq.FP8_ERR_SHAPE
    assert fg(fake, 0, fake, 0, fake, 0, fake, 0, None, 0, 0, None, fake, 2, None, None, 4, 4, 128, None) == sq.FP8_ERR_ARG
    assert fg(fake, 0, fake, 0, fake, 1, fake, 0, None, 0, 0, None, fake, 0, None, None, 4, 4, 128, None) == sq.FP8_ERR_ARG
    assert fg(fake, 0, fake, 0, fake, 0, fake, 0, None, 0, 0, None, fake, 4, None, None, 4, 4, 128, None) == sq.FP8_ERR_DTYPE
    assert fg(fake, 0, fake, 0, fake, 0, fake, 0, fake, 5, 0, None, fake, 0, None, None, 4, 4, 128, None) == sq.FP8_ERR_DTYPE
    c4 = ctypes.c_void_p(0x100004)
    assert fg(fake, 0, fake, 0, fake, 0, fake, 0, None, 0, 0, None, c4, 0, None, None, 4, 4, 128, None) == sq.FP8_ERR_ARG
    assert fg(fake, 0, fake, 0, fake, 0, fake, 2, None, 0, 0, None, fake, 0, None, None, 4, 4, 128, None) == sq.FP8_ERR_ARG
    assert fg(fake, 0, fake, 0, fake, 0, fake, 0, None, 0, 1, None, fake, 2, None, None, 0, 4, 128, None) == sq.FP8_OK
    # layernorm + cast: dtypes, BLOCK granularity, cols not a multiple of the run, cols > 8192,
    # negative eps, missing scale for TENSOR, empty
    ln = lib.fp8_layernorm_quantize
    f1 = ctypes.c_float(1e-5)
    assert ln(fake, 4, 4, 768, fake, None, 1, f1, 0, 0, fake, None, fake, None, None, None, None) == sq.FP8_ERR_DTYPE
    assert ln(fake, 1, 4, 768, fake, None, 6, f1, 0, 0, fake, None, fake, None, None, None, None) == sq.FP8_ERR_DTYPE
    assert ln(fake, 1, 4, 768, fake, None, 1, f1, 0, 2, None, None, fake, fake, None, None, None) == sq.FP8_ERR_ARG
    assert ln(fake, 1, 4, 800, fake, None, 1, f1, 0, 1, None, None, fake, fake, None, None, None) == sq.FP8_ERR_SHAPE
    assert ln(fake, 1, 4, 8320, fake, None, 1, f1, 0, 0, fake, None, fake, None, None, None, None) == sq.FP8_ERR_SHAPE
    assert ln(fake, 1, 4, 768, fake, None, 1, ctypes.c_float(-1.0), 0, 0, fake, None, fake, None, None, None,
              None) == sq.FP8_ERR_ARG
    assert ln(fake, 1, 4, 768, fake, None, 1, f1, 0, 0, None, None, fake, None, None, None, None) == sq.FP8_ERR_ARG
    assert ln(None, 1, 0, 768, None, None, 1, f1, 0, 0, None, None, None, None, None, None, None) == sq.FP8_OK
    # recipe update
    fmts = (ctypes.c_int * 2)(0, 1)
    assert lib.fp8_recipe_update(fake, fake, fake, fmts, 0, 16, 0, 0, None) == sq.FP8_ERR_ARG
    assert lib.fp8_recipe_update(fake, fake, fake, fmts, 2, 16, 1, 0, None) == sq.FP8_ERR_ARG
    assert lib.fp8_recipe_update(fake, fake, fake, fmts, 2, 16, 0, -1, None) == sq.FP8_ERR_ARG
    bad = (ctypes.c_int * 2)(0, 3)
    assert lib.fp8_recipe_update(fake, fake, fake, bad, 2, 16, 0, 0, None) == sq.FP8_ERR_ARG


def test_product_path_does_not_import_oracle():
    """The binding and the HIP sources never reference the oracle package."""
    pkg = os.path.join(ROOT, "scaled_quantize_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU: --gpus 2 exits non-zero with a message, before touching a GPU."""
    import subprocess
    import sys

    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert p.returncode != 0
    assert "one GPU" in p.stderr
