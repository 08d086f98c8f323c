"""Pins of the oracle's LayerNorm + FP8 cast (oracle/layernorm.py): a hand-worked row, the
normalisation invariants, torch's float64 layer_norm as an independent library routine,
the zero-variance row, and hand-derived E4M3 codes."""

import math

import numpy as np
import pytest
import torch

from oracle import fp8 as ofp8, layernorm as oln, quantize as oq


def test_worked_row():
    """[1, 2, 3, 4]: mean 2.5, biased variance 1.25, so y = (x - 2.5) * 2 / sqrt 5."""
    y, mean, rs = oln.layernorm_ref(np.array([[1.0, 2.0, 3.0, 4.0]]), np.ones(4), None, 0.0)
    r5 = math.sqrt(5.0)
    np.testing.assert_allclose(y[0], [-3 / r5, -1 / r5, 1 / r5, 3 / r5], rtol=0, atol=1e-15)
    assert mean[0] == 2.5 and abs(rs[0] - 1 / math.sqrt(1.25)) < 1e-15


def test_invariants():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((6, 768)) * 3 + 1
    eps = 1e-5
    y, mean, rs = oln.layernorm_ref(x, np.ones(768), None, eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-12)
    # shift invariance, positive-scale invariance at eps = 0, affine gamma / beta
    np.testing.assert_allclose(oln.layernorm_ref(x + 100.0, np.ones(768), None, eps)[0], y, atol=1e-10)
    y0 = oln.layernorm_ref(x, np.ones(768), None, 0.0)[0]
    np.testing.assert_allclose(oln.layernorm_ref(x * 7.5, np.ones(768), None, 0.0)[0], y0, atol=1e-12)
    g, b = rng.standard_normal(768), rng.standard_normal(768)
    np.testing.assert_allclose(oln.layernorm_ref(x, g, b, eps)[0], y * g + b, atol=1e-12)


def test_matches_torch_layer_norm_float64():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 256)) * 2
    g, b = rng.standard_normal(256), rng.standard_normal(256)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (256,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    np.testing.assert_allclose(oln.layernorm_ref(x, g, b, 1e-5)[0], want.numpy(), rtol=0, atol=1e-12)


def test_constant_row_gives_beta():
    b = np.linspace(-1, 1, 128)
    y = oln.layernorm_ref(np.full((1, 128), 3.0), np.full(128, 2.0), b, 1e-5)[0]
    assert np.array_equal(y[0], b)


def test_quantized_worked_row():
    """Scale 448 / max|y| on [1, 2, 3, 4]: the ends land on +-448 (0x7E / 0xFE) and +-1/sqrt 5
    at 448 / 3 = 149.3, which rounds to 144 (0x71 / 0xF1) on E4M3's step of 16 above 128."""
    x = np.array([[1.0, 2.0, 3.0, 4.0, 1.0, 2.0, 3.0, 4.0]])
    scale = np.float32(448.0 / (3.0 / math.sqrt(5.0)))
    q, amax = oln.layernorm_quantize(x, np.ones(8), None, 0.0, ofp8.E4M3, oln.TENSOR, scale)
    assert q[0].tolist() == [0xFE, 0xF1, 0x71, 0x7E] * 2
    assert amax == np.float32(3.0 / math.sqrt(5.0))


@pytest.mark.parametrize("gran", [oln.TILE_1x128, oln.MX_1x32])
def test_blockwise_outputs_are_the_quantizers(gran):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    g = rng.standard_normal(256)
    y = oln.layernorm_ref(x, g, None, 1e-5)[0].astype(np.float32)
    got = oln.layernorm_quantize(x, g, None, 1e-5, ofp8.E4M3, gran)
    want = oq.quantize_tile_1x128(y, 0) if gran == oln.TILE_1x128 else oq.quantize_mx_1x32(y, 0)
    assert all(np.array_equal(a, b) for a, b in zip(got, want))
