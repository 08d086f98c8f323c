"""GEMM epilogue reference: bias, GELU or SwiGLU, and an FP8 output with its amax.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the step after the GEMM computes, written out in float64 from the oracle
GEMM's float64 result ``C`` (``oracle.gemm.gemm_ref``):

* bias: ``pre = C + b`` with ``b`` broadcast along rows (the Transformer Engine
  tutorial's module tour builds ``te.Linear(H, H, bias=True)``: Y = X W^T + b);
* GELU in its exact form ``gelu(v) = v * Phi(v)``, Phi the standard normal CDF,
  ``Phi(v) = erfc(-v / sqrt 2) / 2`` (the tutorial's plain-PyTorch block puts
  ``nn.GELU()`` between the MLP's two linears; that module's default is this
  form, not the tanh approximation);
* SwiGLU ``h = silu(g) * u``, ``silu(g) = g * sigmoid(g) = g / (1 + e^-g)``
  (the course page's MoE exercise sizes a SwiGLU expert at 3 D F parameters:
  gate, up and down projections).  R (layout reading; the pages give none): the
  pre-activation's columns interleave the two projections, column 2f is gate
  unit f and column 2f+1 its up unit, so h has half the columns;
* FP8 output for the next layer's input: the per-tensor quantizer of
  ``oracle.quantize`` applied to the activation output (codes
  ``enc(fp32(y * scale))``, amax = max |y| in float32), the lesson's Part 01
  rule that every FP8 tensor's amax is recorded.

``erfc`` is scipy's (a library routine standing in for one step).
"""

from __future__ import annotations

import numpy as np
from scipy import special

from . import quantize

ACT_NONE, ACT_GELU, ACT_SWIGLU = 0, 1, 2


def gelu(v) -> np.ndarray:
    """v * Phi(v) in float64."""
    v = np.asarray(v, dtype=np.float64)
    return v * 0.5 * special.erfc(-v / np.sqrt(2.0))


def silu(g) -> np.ndarray:
    """g / (1 + e^-g) in float64 (e^-g overflowing to inf gives -0 / 0, the limit)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(pre) -> np.ndarray:
    """[rows][2F] interleaved (gate, up) columns -> [rows][F] silu(gate) * up."""
    pre = np.asarray(pre, dtype=np.float64)
    assert pre.shape[-1] % 2 == 0, "SwiGLU needs an even number of columns"
    return silu(pre[..., 0::2]) * pre[..., 1::2]


def epilogue_ref(C, bias=None, act=ACT_NONE):
    """(pre, y): the pre-activation C + bias and the activation output, float64."""
    pre = np.asarray(C, dtype=np.float64)
    if bias is not None:
        pre = pre + np.asarray(bias, dtype=np.float64)[None, :]
    if act == ACT_NONE:
        return pre, pre
    if act == ACT_GELU:
        return pre, gelu(pre)
    if act == ACT_SWIGLU:
        return pre, swiglu(pre)
    raise ValueError("act")


def fp8_output(y, scale, fmt):
    """The activation output quantised for the next layer: (codes, amax)."""
    with np.errstate(over="ignore"):
        return quantize.quantize_tensor(np.asarray(y, dtype=np.float64).astype(np.float32), scale, fmt)
