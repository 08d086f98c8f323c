"""Symmetric int8 absmax quantisation: the course page's worked example.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Week 14" course page, absmax paragraph: the grid step is
step = max|x| / (2^(b-1) - 1), q = round(x / step), x ~ q * step; the scale can
be per tensor or per block.  This is the integer analogue of the FP8 scale rule
(there the scale is a multiplier that sends amax to the format's largest value;
here the step sends amax to 127).  It is not on the FP8 path; it checks the
amax -> scale -> round building blocks against the numbers the page prints.
Rounding of exact halves is to even (R: the page's examples contain no ties).
"""

from __future__ import annotations

import numpy as np


def absmax_quantize(x, bits: int = 8):
    """Per-tensor absmax: (q int64, step, dequantised float64)."""
    x = np.asarray(x, dtype=np.float64)
    qmax = 2 ** (bits - 1) - 1
    step = np.abs(x).max() / qmax
    q = np.rint(x / step).astype(np.int64)
    return q, step, q * step


def absmax_quantize_blocks(x, block: int, bits: int = 8):
    """Per-block absmax over consecutive runs of ``block`` elements -> (q, steps)."""
    x = np.asarray(x, dtype=np.float64)
    qmax = 2 ** (bits - 1) - 1
    xb = x.reshape(-1, block)
    steps = np.abs(xb).max(axis=1) / qmax
    q = np.rint(xb / steps[:, None]).astype(np.int64).reshape(x.shape)
    return q, steps
