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


# ------------------------------------------------------------------ binding buffer checks
#
# The C side sees only pointers, so the binding checks every caller-supplied tensor's dtype,
# shape and contiguity, then that all of a call's tensors are on one GPU, before anything
# reaches the library.  On the CPU every check runs in that order: a mis-sized buffer raises
# its own error; correctly sized host tensors end at the device check.


def _e(*shape, dtype=None):
    import torch

    return torch.empty(shape, dtype=dtype or torch.float32)


def _raises(fn, exc, match):
    with pytest.raises(exc, match=match):
        fn()


def test_gemm_rejects_mis_sized_buffers():
    import torch

    import scaled_quantize_gemm_amd as sq

    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    M, N, K = 64, 48, 256
    A, B = _e(M, K, dtype=u8), _e(N, K, dtype=u8)
    one = _e(1)
    g = sq.fp8_gemm
    _raises(lambda: g(A.float(), 0, one, 0, B, 0, one, 0), TypeError, "A must be")
    _raises(lambda: g(A, 0, one, 0, _e(N, K + 128, dtype=u8), 0, one, 0), ValueError, "K mismatch")
    _raises(lambda: g(A, 0, one, 0, B, 0, one, 0, sq.OUT_F32, C=_e(M, N, dtype=bf)), TypeError, "C must be")
    _raises(lambda: g(A, 0, one, 0, B, 0, one, 0, sq.OUT_BF16, C=_e(M, N - 1, dtype=bf)), ValueError, "C must have")
    _raises(lambda: g(A, 0, one, 0, B, 0, one, 0, sq.OUT_F32, C=_e(N, M).t()), ValueError, "contiguous")
    _raises(lambda: g(A, 0, _e(0), 0, B, 0, one, 0), ValueError, "at least 1")
    _raises(lambda: g(A, 0, one.double(), 0, B, 0, one, 0), TypeError, "a_scale_inv must be")
    # TILE x BLOCK: [K/128][M] and [ceil(N/128)][K/128]
    sa, sb = _e(K // 128, M), _e(1, K // 128)
    _raises(lambda: g(A, 0, _e(K // 128, M - 1), 1, B, 0, sb, 2), ValueError, "a_scale_inv must have")
    _raises(lambda: g(A, 0, sa, 1, B, 0, _e(K // 128, 1), 2), ValueError, "b_scale_inv must have")
    # TILE x TILE: B's scales [K/128][N]
    _raises(lambda: g(A, 0, sa, 1, B, 0, _e(K // 128, N + 1), 1), ValueError, "b_scale_inv must have")
    # MX: uint8 [K/32][rows]
    _raises(lambda: g(A, 0, _e(K // 32, M), 3, B, 0, _e(K // 32, N, dtype=u8), 3), TypeError, "a_scale_inv must be")
    _raises(lambda: g(A, 0, _e(M, K // 32, dtype=u8), 3, B, 0, _e(K // 32, N, dtype=u8), 3), ValueError,
            "a_scale_inv must have")
    _raises(lambda: g(A, 0, one, 0, B, 0, one, 0, sq.OUT_E4M3), ValueError, "OUT_F32 or OUT_BF16")
    # every size right: the host tensors stop at the device check
    _raises(lambda: g(A, 0, sa, 1, B, 0, sb, 2, sq.OUT_BF16, C=_e(M, N, dtype=bf)), ValueError, "GPU tensor")


def test_fused_gemm_rejects_mis_sized_buffers():
    import torch

    import scaled_quantize_gemm_amd as sq

    u8, bf = torch.uint8, torch.bfloat16
    M, N, K = 32, 64, 128
    A, B, one = _e(M, K, dtype=u8), _e(N, K, dtype=u8), _e(1)
    f = sq.fp8_gemm_fused
    _raises(lambda: f(A, 0, one, 0, B, 0, one, 0, sq.OUT_BF16, act=sq.FP8_ACT_SWIGLU, C=_e(M, N, dtype=bf)),
            ValueError, "C must have")
    _raises(lambda: f(A, 0, one, 0, B, 0, one, 0, sq.OUT_E4M3, C=_e(M, N, dtype=bf)), TypeError, "C must be")
    _raises(lambda: f(A, 0, one, 0, B, 0, one, 0, sq.OUT_BF16, aux=_e(M, N)), TypeError, "aux must be")
    _raises(lambda: f(A, 0, one, 0, B, 0, one, 0, sq.OUT_BF16, aux=_e(M, N // 2, dtype=bf)), ValueError,
            "aux must have")
    _raises(lambda: f(A, 0, one, 0, B, 0, one, 0, sq.OUT_BF16, bias=_e(N + 1)), ValueError, "bias must have")
    _raises(lambda: f(A, 0, one, 0, B, 0, one, 0, sq.OUT_E4M3, c_scale=_e(0), c_amax=one), ValueError, "at least 1")
    _raises(lambda: f(A, 0, one, 0, B, 0, one, 0, sq.OUT_E4M3, c_scale=one, c_amax=one), ValueError, "GPU tensor")


def test_casts_reject_mis_sized_buffers():
    import torch

    import scaled_quantize_gemm_amd as sq

    u8, bf, f32 = torch.uint8, torch.bfloat16, torch.float32
    x = _e(256, 384, dtype=bf)
    one = _e(1)
    _raises(lambda: sq.fp8_quantize(x.half(), 0), TypeError, "x must be")
    _raises(lambda: sq.fp8_quantize(x, 0, q=_e(256, 383, dtype=u8)), ValueError, "q must have")
    _raises(lambda: sq.fp8_quantize(x, 0, 1, scale_inv_out=_e(256, 3)), ValueError, "scale_inv_out must have")
    _raises(lambda: sq.fp8_quantize(x, 0, 2, scale_inv_out=_e(3, 2)), ValueError, "scale_inv_out must have")
    _raises(lambda: sq.fp8_quantize(x, 0, 3, scale_inv_out=_e(12, 256)), TypeError, "scale_inv_out must be")
    _raises(lambda: sq.fp8_quantize(x, 0, 0, scale=_e(1, dtype=bf)), TypeError, "scale must be")
    _raises(lambda: sq.fp8_quantize(x, 0, 0, scale=one, amax_slot=_e(0)), ValueError, "at least 1")
    _raises(lambda: sq.fp8_quantize(x, 0, 0, scale=one), ValueError, "GPU tensor")
    _raises(lambda: sq.fp8_quantize_diag(x, 0, one, _e(2, dtype=torch.int64)), ValueError, "counts must have")
    _raises(lambda: sq.fp8_cast_transpose(x, 0, one, qT=_e(256, 384, dtype=u8)), ValueError, "qT must have")
    _raises(lambda: sq.fp8_cast_transpose(x, 0, one, q=_e(384, 256, dtype=u8)), ValueError, "q must have")
    _raises(lambda: sq.fp8_cast_transpose_blockwise(x, 0, 1, q_scale_inv=_e(2, 256)), ValueError,
            "q_scale_inv must have")
    _raises(lambda: sq.fp8_cast_transpose_blockwise(x, 0, 2, qT_scale_inv=_e(2, 3)), ValueError,
            "qT_scale_inv must have")
    g = _e(384, dtype=bf)
    _raises(lambda: sq.fp8_layernorm_quantize(x, _e(383, dtype=bf), None, 1e-5, 0), ValueError, "gamma must have")
    _raises(lambda: sq.fp8_layernorm_quantize(x, g, _e(384), 1e-5, 0), TypeError, "beta must be")
    _raises(lambda: sq.fp8_layernorm_quantize(x, g, None, 1e-5, 0, mu=_e(255)), ValueError, "mu must have")
    _raises(lambda: sq.fp8_layernorm_quantize(x, g, None, 1e-5, 0, 1, scale_inv_out=_e(3, 255)), ValueError,
            "scale_inv_out must have")
    _raises(lambda: sq.fp8_recipe_update(_e(16, 3), _e(2), _e(3), [0, 0, 1]), ValueError, "scale must have")
    _raises(lambda: sq.fp8_recipe_update(_e(16, 3), _e(3), _e(3), [0, 0, 1]), ValueError, "GPU tensor")


def test_calibration_library_exports_its_header():
    """include/fp8_calib.h (the measurement kernels bench.py loads) against libfp8calib.so."""
    from scaled_quantize_gemm_amd.build import CALIB_LIBNAME, LIBDIR

    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "fp8_calib.h")).read(), flags=re.S)
    names = re.findall(r"^\s*(?:int|double)\s+(fp8_calib_\w+)\s*\(", src, re.M)
    assert sorted(names) == ["fp8_calib_mfma", "fp8_calib_mfma_flops", "fp8_calib_wall_clock_khz"]
    lib = ctypes.CDLL(os.path.join(LIBDIR, CALIB_LIBNAME))
    for name in names:
        assert hasattr(lib, name), name
    lib.fp8_calib_mfma_flops.restype = ctypes.c_double
    assert lib.fp8_calib_mfma_flops(2, 3) == 2 * 8 * 3 * 16 * 2.0 * 32 * 32 * 64
