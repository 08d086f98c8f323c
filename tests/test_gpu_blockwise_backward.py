"""GPU parity of the blockwise backward pieces against the oracle: the blockwise
cast-transpose (1x128 runs along the new K for X^T and dY^T, transposed 128x128 blocks for
W^T; codes and scales bit-exact) and the TILE_1x128 x TILE_1x128 GEMM (wgrad), then a
whole layer's forward, dgrad and wgrad with E4M3 everywhere."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import DEV, announce, assert_codes_equal, assert_f32_bits_equal, check_gemm, f32_np, np_of  # noqa: E402
from oracle import fp8 as ofp8, gemm as og, quantize as oq  # noqa: E402
import workloads  # noqa: E402

TILE, BLOCK = 1, 2


@pytest.fixture(scope="module")
def sq():
    import scaled_quantize_gemm_amd as m

    ok, why = m.fp8_device_check(0)
    assert ok, why
    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _data(rows, cols, seed, specials=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-12, 12, (rows, 1))).astype(np.float32)
    x *= np.exp2(rng.integers(-6, 6, (1, cols))).astype(np.float32)
    if specials:
        x[0:128, 3] = 0.0  # a zero column run and zero entries in every row run it crosses
        x[5, 0:128] = 0.0  # a zero row run
        x[7, 9] = np.nan
        x[9, 130 % cols] = np.inf
        x[11, 2] = -0.0
        x[13, 4] = 1e-41
        x[17, 6] *= 1e4
    return x


@pytest.mark.parametrize("gran", [TILE, BLOCK])
@pytest.mark.parametrize("fmt", [ofp8.E4M3, ofp8.E5M2])
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 1024), (1024, 512)])
def test_cast_transpose_blockwise(sq, gran, fmt, bf16, shape):
    announce("cast_transpose_blockwise", gran, ofp8.fmt_name(fmt), "bf16" if bf16 else "f32", shape)
    x = _data(*shape, seed=shape[0] + 5 * shape[1] + gran)
    xt = torch.from_numpy(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
    q, qs, qT, qTs = sq.fp8_cast_transpose_blockwise(xt.to(DEV), fmt, gran)
    torch.cuda.synchronize()
    oq_, oqs, oqT, oqTs = oq.cast_transpose_blockwise(f32_np(xt), fmt, gran)
    assert_codes_equal(np_of(q), oq_, "q")
    assert_f32_bits_equal(np_of(qs), oqs, "q scale_inv")
    assert_codes_equal(np_of(qT), oqT, "qT")
    assert_f32_bits_equal(np_of(qTs), oqTs, "qT scale_inv")


def _tile_operands(rng, M, N, K):
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp2(rng.integers(-6, 6, (M, 1))).astype(np.float32)
    y = rng.standard_normal((N, K)).astype(np.float32) * np.exp2(rng.integers(-6, 6, (N, 1))).astype(np.float32)
    y[:, :128] *= 30.0
    A, sa = oq.quantize_tile_1x128(x, 0)
    B, sb = oq.quantize_tile_1x128(y, 0)
    return A, sa, B, sb


@pytest.mark.parametrize("out", [0, 1])
@pytest.mark.parametrize("mnk", [(256, 256, 256), (200, 300, 512), (1, 130, 128), (129, 257, 384)])
def test_tile_by_tile_gemm_small(sq, out, mnk):
    M, N, K = mnk
    announce("tile x tile gemm", out, mnk)
    rng = np.random.default_rng(M + 7 * N + K)
    A, sa, B, sb = _tile_operands(rng, M, N, K)
    C = sq.fp8_gemm(_t(A), 0, _t(sa), TILE, _t(B), 0, _t(sb), TILE, out)
    torch.cuda.synchronize()
    Cr, S, G = og.gemm_ref(A, 0, sa, og.TILE_1x128, B, 0, sb, og.TILE_1x128)
    check_gemm(np_of(C), Cr, S, G, K, "block", out == 1, f"tile x tile {mnk} out{out}")


@pytest.mark.parametrize("out", [0, 1])
@pytest.mark.parametrize("mnk", [(2085, 4100, 384), (2048, 4097, 1152), (1300, 3000, 128), (300, 520, 14336)])
def test_tile_by_tile_gemm_large(sq, out, mnk):
    M, N, K = mnk
    announce("large tile x tile gemm", out, mnk)
    rng = np.random.default_rng(M + 11 * N + K)
    A, sa, B, sb = _tile_operands(rng, M, N, K)
    C = sq.fp8_gemm(_t(A), 0, _t(sa), TILE, _t(B), 0, _t(sb), TILE, out)
    torch.cuda.synchronize()
    r = np.sort(rng.choice(M, 160, replace=False))
    r[-1] = M - 1
    Cr, S, G = og.gemm_ref(A, 0, sa, og.TILE_1x128, B, 0, sb, og.TILE_1x128, rows=r)
    check_gemm(np_of(C)[r], Cr, S, G, K, "block", out == 1, f"large tile x tile {mnk} out{out}")


def test_blockwise_layer_forward_and_backward(sq):
    """Workload-3 style layer at reduced size (tokens 2048, in 2048, out 4096), E4M3 everywhere:
    forward Y = X W^T (TILE x BLOCK), dgrad dX = dY W (A = dY in 1x128 runs along the output
    features, B = W^T in transposed blocks), wgrad dW = dY^T X (A = dY^T and B = X^T, both in
    1x128 runs along the tokens)."""
    M, K, N = 2048, 2048, 4096
    X, W = workloads.w3_inputs(m=M, k=K, n=N)
    dY = workloads.w3_grad(m=M, n=N)
    rng = np.random.default_rng(3)
    xd, wd, gd = X.to(DEV), W.to(DEV), dY.to(DEV)
    announce("blockwise layer: quantize")
    qX, sX, qXT, sXT = sq.fp8_cast_transpose_blockwise(xd, 0, TILE)
    qW, sW, qWT, sWT = sq.fp8_cast_transpose_blockwise(wd, 0, BLOCK)
    qG, sG, qGT, sGT = sq.fp8_cast_transpose_blockwise(gd, 0, TILE)
    announce("blockwise layer: gemms")
    Y = sq.fp8_gemm(qX, 0, sX, TILE, qW, 0, sW, BLOCK, sq.OUT_BF16)
    dX = sq.fp8_gemm(qG, 0, sG, TILE, qWT, 0, sWT, BLOCK, sq.OUT_BF16)
    dW = sq.fp8_gemm(qGT, 0, sGT, TILE, qXT, 0, sXT, TILE, sq.OUT_BF16)
    torch.cuda.synchronize()
    announce("blockwise layer: oracle quantization")
    oX = oq.cast_transpose_blockwise(f32_np(X), 0, TILE)
    oW = oq.cast_transpose_blockwise(f32_np(W), 0, BLOCK)
    oG = oq.cast_transpose_blockwise(f32_np(dY), 0, TILE)
    for got, want, name in [((qX, sX, qXT, sXT), oX, "X"), ((qW, sW, qWT, sWT), oW, "W"),
                            ((qG, sG, qGT, sGT), oG, "dY")]:
        assert_codes_equal(np_of(got[0]), want[0], f"{name} q")
        assert_f32_bits_equal(np_of(got[1]), want[1], f"{name} q scale_inv")
        assert_codes_equal(np_of(got[2]), want[2], f"{name} qT")
        assert_f32_bits_equal(np_of(got[3]), want[3], f"{name} qT scale_inv")
    announce("blockwise layer: oracle gemms (sampled rows)")
    for C, (A, sa, ga), (B, sb, gb), rows, label in [
            (Y, (oX[0], oX[1], og.TILE_1x128), (oW[0], oW[1], og.BLOCK_128x128), M, "forward"),
            (dX, (oG[0], oG[1], og.TILE_1x128), (oW[2], oW[3], og.BLOCK_128x128), M, "dgrad"),
            (dW, (oG[2], oG[3], og.TILE_1x128), (oX[2], oX[3], og.TILE_1x128), N, "wgrad")]:
        r = np.sort(rng.choice(rows, 96, replace=False))
        Cr, S, G = og.gemm_ref(A, 0, sa, ga, B, 0, sb, gb, rows=r)
        check_gemm(np_of(C)[r], Cr, S, G, A.shape[1], "block", True, f"blockwise layer {label}")
