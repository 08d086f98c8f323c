"""amax and scale derivation: delayed scaling (amax-history ring), current blockwise scaling, MX e8m0.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

amax ("Transformer Scaling" lesson, Core vocabulary: the largest absolute value
in a tensor or in a history window):

* computed in float32 over the granule; -0 counts as 0;
* R (reading, the pages are silent): a NaN anywhere makes the amax NaN.

Scale (lesson, Part 01: a scale maps source values into the FP8 range, often
using amax; Worked example 01: scale = 448 / 240, so the amax lands on the
largest E4M3 value).  The scale is a multiplier, ``q = enc(x * scale)``, and
``scale_inv = 1 / scale`` is the dequantisation step.

Delayed scaling (lesson, Part 01 and Core vocabulary: the scale comes from the
amax history, which avoids a pre-quantisation read at the price of lag; the
Transformer Engine tutorial's recipe: amax_history_len=16,
amax_compute_algo="max", and its readback ``amax_history[0, :4]``, which makes
the history a [length, tensors] array).  Readings (R) where the pages leave the
mechanics open:

* R: initial state: history all zero, scale = scale_inv = 1;
* each quantisation of tensor slot j max-es its amax into ``hist[0][j]``;
* after the step, the update: m_j = max_i hist[i][j] ("max" algorithm).  If m_j
  is finite and > 0: scale_j = fp32(fp32(fmax / m_j) * 2^-margin), clamped to
  the largest finite float32 if it overflows (R), and
  scale_inv_j = fp32(1 / scale_j) (R: stored as the reciprocal of the scale);
  otherwise (m_j zero, inf or NaN) both keep their previous values (R);
* roll: hist[i] <- hist[i + 1] for i < H - 1, hist[H - 1] <- old hist[0], then
  hist[0] <- 0.  An amax recorded at step t therefore enters the scales of
  steps t+1 .. t+H and no other.

Current blockwise scaling (week-14 course page, absmax paragraph: DeepSeek-V3
scales every 128 activation values and every 128 x 128 weight block, computing
the scale from the current block "online"):

* s = fp32(fmax / amax_block), clamped to the largest finite float32 (R);
  scale_inv = fp32(1 / s);
* R: a block whose amax is zero or not finite gets s = scale_inv = 1.

MX (same paragraph: MX formats give every 32 numbers a shared scale):

* R: the shared scale is a power of two 2^E stored as e8m0 code E + 127, with
  E the smallest integer such that amax_group <= fmax * 2^E (the group maximum
  lands in (fmax/2, fmax] and nothing clips -- the pages treat clipping as the
  failure mode to avoid); E is clamped to [-127, 127], so an all-zero group
  gets code 0; a group whose amax is not finite gets code 255 (NaN).
"""

from __future__ import annotations

import numpy as np

from .fp8 import FMAX

FLT_MAX = np.float32(np.finfo(np.float32).max)


def amax(x) -> np.float32:
    """max |x| in float32 (NaN-propagating; 0 for an empty input)."""
    a = np.abs(np.asarray(x, dtype=np.float32))
    if a.size == 0:
        return np.float32(0.0)
    if np.isnan(a).any():
        return np.float32(np.nan)
    return np.float32(a.max())


def _ratio(fmax: float, m) -> np.ndarray:
    """fp32(fmax / m), overflow clamped to FLT_MAX."""
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        r = np.float32(fmax) / np.asarray(m, dtype=np.float32)
    return np.where(np.isinf(r), FLT_MAX, r).astype(np.float32)


def _recip(s) -> np.ndarray:
    with np.errstate(divide="ignore", over="ignore"):
        return (np.float32(1.0) / np.asarray(s, dtype=np.float32)).astype(np.float32)


# --------------------------------------------------------------------------- delayed scaling


class DelayedState:
    """Amax-history ring and per-slot scales of the delayed-scaling recipe."""

    def __init__(self, n_slots: int, history_len: int):
        self.hist = np.zeros((history_len, n_slots), dtype=np.float32)
        self.scale = np.ones(n_slots, dtype=np.float32)
        self.scale_inv = np.ones(n_slots, dtype=np.float32)

    def copy(self) -> "DelayedState":
        c = DelayedState(self.hist.shape[1], self.hist.shape[0])
        c.hist[...] = self.hist
        c.scale[...] = self.scale
        c.scale_inv[...] = self.scale_inv
        return c

    def record(self, slot: int, a) -> None:
        """hist[0][slot] = max(hist[0][slot], a) with NaN propagating."""
        self.hist[0, slot] = np.float32(np.maximum(self.hist[0, slot], np.float32(a)))


def delayed_update(state: DelayedState, fmts, margin: int = 0) -> DelayedState:
    """One end-of-step update of every slot; returns a new state."""
    out = state.copy()
    with np.errstate(invalid="ignore"):
        m = state.hist.max(axis=0)  # NaN-propagating max over the window
    for j, fmt in enumerate(fmts):
        mj = np.float32(m[j])
        if np.isfinite(mj) and mj > 0:
            s = _ratio(FMAX[fmt], mj)
            s = np.float32(s * np.float32(2.0 ** -margin))
            out.scale[j] = s
            out.scale_inv[j] = _recip(s)
    out.hist = np.roll(state.hist, -1, axis=0)
    out.hist[0, :] = 0.0
    return out


# --------------------------------------------------------------------------- current scaling


def current_scale(block_amax, fmt):
    """Per-block (scale, scale_inv) from block amaxes; zero / non-finite blocks get 1."""
    a = np.asarray(block_amax, dtype=np.float32)
    ok = np.isfinite(a) & (a > 0)
    s = np.where(ok, _ratio(FMAX[fmt], np.where(ok, a, 1.0)), np.float32(1.0)).astype(np.float32)
    s_inv = np.where(ok, _recip(s), np.float32(1.0)).astype(np.float32)
    return s, s_inv


# --------------------------------------------------------------------------- MX e8m0


def mx_exponent(group_amax, fmt) -> np.ndarray:
    """e8m0 codes: smallest E with amax <= fmax * 2^E, clamped to [-127, 127]; 255 if not finite."""
    g = np.asarray(group_amax, dtype=np.float32).astype(np.float64)
    fmax = FMAX[fmt]
    finite = np.isfinite(g)
    gg = np.where(finite & (g > 0), g, 1.0)
    # start from an estimate and correct it with exact power-of-two comparisons
    e = np.ceil(np.log2(gg / fmax)).astype(np.int64)
    e = np.where(gg > fmax * np.exp2(e.astype(np.float64)), e + 1, e)
    e = np.where(gg <= fmax * np.exp2((e - 1).astype(np.float64)), e - 1, e)
    e = np.where(g > 0, e, -127)
    e = np.clip(e, -127, 127)
    code = (e + 127).astype(np.uint8)
    return np.where(finite, code, np.uint8(255)).astype(np.uint8)
