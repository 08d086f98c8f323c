"""LayerNorm followed by the FP8 cast of its output (the step before the FP8 linear).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The Transformer Engine tutorial's module tour builds te.LayerNorm,
te.LayerNormLinear and te.LayerNormMLP, and its plain-PyTorch block applies
nn.LayerNorm before attention and before the MLP.  The definition, written out
per row of x [rows][cols] in float64:

    mean  = sum_j x_j / cols
    var   = sum_j (x_j - mean)^2 / cols          (biased: divide by cols)
    rs    = 1 / sqrt(var + eps)
    y_j   = (x_j - mean) * rs * gamma_j + beta_j  (beta omitted: no shift)

R (reading; the pages name the module, not its constants): eps is the
caller's, nn.LayerNorm's default being 1e-5.

The FP8 output is the pinned quantizer of ``oracle.quantize`` applied to y
rounded to float32 (the precision the cast sees): per tensor with a delayed
scale (plus amax), 1x128 runs, or MX 1x32 runs.
"""

from __future__ import annotations

import numpy as np

from . import quantize

TENSOR, TILE_1x128, MX_1x32 = 0, 1, 3


def layernorm_ref(x, gamma, beta, eps):
    """(y, mean, rs) in float64; y [rows][cols], mean and rs [rows]."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.sum(axis=1) / x.shape[1]
    d = x - mean[:, None]
    var = (d * d).sum(axis=1) / x.shape[1]
    rs = 1.0 / np.sqrt(var + np.float64(eps))
    y = d * rs[:, None] * np.asarray(gamma, dtype=np.float64)[None, :]
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)[None, :]
    return y, mean, rs


def layernorm_quantize(x, gamma, beta, eps, fmt, granularity, scale=None):
    """LayerNorm, then the quantizer of `granularity` on fp32(y).

    TENSOR -> (q, amax) with the given scale; TILE_1x128 -> (q, scale_inv [cols/128][rows]);
    MX_1x32 -> (q, e8m0 [rows][cols/32])."""
    y = layernorm_ref(x, gamma, beta, eps)[0]
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)
    if granularity == TENSOR:
        return quantize.quantize_tensor(y32, np.float32(scale), fmt)
    if granularity == TILE_1x128:
        return quantize.quantize_tile_1x128(y32, fmt)
    if granularity == MX_1x32:
        return quantize.quantize_mx_1x32(y32, fmt)
    raise ValueError("granularity")
