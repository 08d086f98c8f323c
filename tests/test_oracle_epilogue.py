"""Pins of the oracle's GEMM epilogue (oracle/epilogue.py): tabulated values of the standard
normal CDF, closed forms and identities of GELU and SiLU, brute force for bias and the
interleaved SwiGLU layout, and the FP8 output against the pinned per-tensor quantizer."""

import math

import numpy as np
import pytest

from oracle import epilogue as oe, fp8 as ofp8, gemm as og, quantize as oq

# Standard normal CDF at 0.5, 1, 2, 3 as printed in statistical tables (to 15 digits).
PHI_TABLE = {0.5: 0.691462461274013, 1.0: 0.841344746068543, 2.0: 0.977249868051821, 3.0: 0.998650101968370}


@pytest.mark.parametrize("x", sorted(PHI_TABLE))
def test_gelu_is_x_times_normal_cdf(x):
    """gelu(x) = x Phi(x) and gelu(-x) = -x (1 - Phi(x)): a dropped 1/sqrt 2 in the erfc
    argument, or the tanh approximation, misses these by > 1e-4."""
    assert abs(oe.gelu(x) - x * PHI_TABLE[x]) < 1e-14
    assert abs(oe.gelu(-x) - (-x) * (1.0 - PHI_TABLE[x])) < 1e-14


def test_gelu_identities():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000) * 4
    # x Phi(x) - (-x) Phi(-x) = x (Phi(x) + Phi(-x)) = x
    np.testing.assert_allclose(oe.gelu(x) - oe.gelu(-x), x, rtol=0, atol=1e-14)
    assert oe.gelu(0.0) == 0.0
    assert oe.gelu(40.0) == 40.0  # Phi(40) = 1 in float64
    assert oe.gelu(-40.0) == pytest.approx(0.0, abs=1e-300)
    # tiny x: Phi(x) -> 1/2
    assert oe.gelu(1e-30) == pytest.approx(0.5e-30, rel=1e-15)


def test_silu_closed_forms():
    # silu(1) = sigmoid(1) = e / (1 + e); silu(0) = 0; silu(x) - silu(-x) = x
    assert abs(oe.silu(1.0) - math.e / (1.0 + math.e)) < 1e-16
    assert oe.silu(0.0) == 0.0
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000) * 6
    np.testing.assert_allclose(oe.silu(x) - oe.silu(-x), x, rtol=0, atol=1e-13)
    # large |x|: silu -> x and -> -0
    assert oe.silu(800.0) == 800.0
    v = oe.silu(-800.0)
    assert v == 0.0 and math.copysign(1.0, v) == -1.0


def _brute_linear(a, b, bias):
    """Pure-Python Y[m][n] = sum_k a[m][k] b[n][k] + bias[n]."""
    M, K = len(a), len(a[0])
    N = len(b)
    return [[sum(a[m][k] * b[n][k] for k in range(K)) + (bias[n] if bias is not None else 0.0) for n in range(N)]
            for m in range(M)]


def test_bias_and_swiglu_layout_by_brute_force():
    """Gate and up weights interleaved into B (row 2f = gate f, row 2f+1 = up f) give
    silu(X Wg^T + bg) * (X Wu^T + bu), computed here by loops over the decoded values."""
    rng = np.random.default_rng(2)
    M, F, K = 3, 4, 128
    x = rng.standard_normal((M, K)).astype(np.float32)
    wg = (rng.standard_normal((F, K)) * 0.1).astype(np.float32)
    wu = (rng.standard_normal((F, K)) * 0.1).astype(np.float32)
    bg, bu = rng.standard_normal(F), rng.standard_normal(F)
    w = np.empty((2 * F, K), np.float32)
    w[0::2], w[1::2] = wg, wu
    b = np.empty(2 * F)
    b[0::2], b[1::2] = bg, bu
    sx, sw = np.float32(448.0 / np.abs(x).max()), np.float32(448.0 / np.abs(w).max())
    qa, qb = oq.quantize_tensor(x, sx, 0)[0], oq.quantize_tensor(w, sw, 0)[0]
    sa, sb = np.float32(1.0) / sx, np.float32(1.0) / sw
    C = og.gemm_ref(qa, 0, sa, og.TENSOR, qb, 0, sb, og.TENSOR)[0]
    pre, y = oe.epilogue_ref(C, b, oe.ACT_SWIGLU)
    ad = (ofp8.decode(qa, 0) * np.float64(sa)).tolist()
    bd = (ofp8.decode(qb, 0) * np.float64(sb)).tolist()
    gate = _brute_linear(ad, bd[0::2], list(bg))
    up = _brute_linear(ad, bd[1::2], list(bu))
    want = [[gate[m][f] / (1.0 + math.exp(-gate[m][f])) * up[m][f] for f in range(F)] for m in range(M)]
    assert y.shape == (M, F)
    np.testing.assert_allclose(y, np.array(want), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(pre, np.array(_brute_linear(ad, bd, list(b))), rtol=1e-12, atol=1e-12)


def test_gelu_and_none_epilogues():
    rng = np.random.default_rng(3)
    C = rng.standard_normal((5, 6))
    bias = rng.standard_normal(6)
    pre, y = oe.epilogue_ref(C, bias, oe.ACT_NONE)
    assert np.array_equal(pre, C + bias) and np.array_equal(y, pre)
    pre, y = oe.epilogue_ref(C, None, oe.ACT_GELU)
    assert np.array_equal(pre, C)
    for (i, j), v in np.ndenumerate(C):
        assert abs(y[i, j] - v * 0.5 * math.erfc(-v / math.sqrt(2.0))) < 1e-15


def test_fp8_output_is_the_per_tensor_quantizer():
    """Codes and amax of the output equal the pinned per-tensor quantizer's; values past
    fmax / scale saturate (the lesson's clip at 448)."""
    rng = np.random.default_rng(4)
    y = rng.standard_normal((7, 9)) * 3
    y[0, 0] = 1000.0
    y[1, 1] = -1000.0
    for fmt in (ofp8.E4M3, ofp8.E5M2):
        scale = np.float32(ofp8.FMAX[fmt] / 8.0)
        q, amax = oe.fp8_output(y, scale, fmt)
        q2, amax2 = oq.quantize_tensor(y.astype(np.float32), scale, fmt)
        assert np.array_equal(q, q2) and amax == amax2 == np.float32(1000.0)
        top = 0x7E if fmt == ofp8.E4M3 else 0x7B
        assert q[0, 0] == top and q[1, 1] == (0x80 | top)
