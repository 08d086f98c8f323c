"""Running sums kept in FP8, with and without promotion to fp32.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Week 14" course page, accumulation-precision bullet: in E4M3 the spacing in
[64, 128) is 8, so 64 + 3 = 64; adding 100 threes with the running sum rounded
to E4M3 after every addition gets stuck at 64 after 18 steps; promoting the
partial sum to fp32 every 8 terms gives exactly 300.

R (reading): at each promotion the FP8 partial sum is added to an fp32 total
and restarts from zero; additions inside an interval round to the FP8 format
(nearest, ties to even, saturating) after every step.
"""

from __future__ import annotations

import numpy as np

from . import fp8


def _round(v: float, fmt: int) -> float:
    return float(fp8.decode(fp8.encode(np.float32(v), fmt), fmt))


def fp8_running_sum(terms, fmt: int = fp8.E4M3, trace: bool = False):
    """Sum with the partial sum rounded to FP8 after each addition."""
    s = 0.0
    hist = []
    for t in terms:
        s = _round(s + float(t), fmt)
        hist.append(s)
    return (s, hist) if trace else s


def promoted_sum(terms, interval: int, fmt: int = fp8.E4M3) -> float:
    """FP8 partial sums over runs of ``interval`` terms, each promoted into an fp32 total."""
    total = np.float32(0.0)
    partial = 0.0
    for i, t in enumerate(terms, 1):
        partial = _round(partial + float(t), fmt)
        if i % interval == 0:
            total = np.float32(total + np.float32(partial))
            partial = 0.0
    return float(np.float32(total + np.float32(partial)))
