"""FP8 (OCP E4M3 / E5M2), bf16 and e8m0 number formats, written from their definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Formats ("Transformer Scaling" lesson, Concept deep dive 01; week-14 course page,
FP8 bullet: E4M3 = 4 exponent + 3 mantissa bits, max 448; E5M2 = 5 + 2 bits,
max 57,344):

* E4M3: bias 7.  The printed maximum 448 = 1.75 * 2^8 can only be reached if the
  all-ones exponent field holds finite values, so the layout is the one where
  only S.1111.111 is NaN and there is no infinity.  Subnormals m/8 * 2^-6.
* E5M2: bias 15, IEEE-like.  57,344 = 1.75 * 2^15 is the largest value below
  the all-ones exponent, which holds +-inf (mantissa 0) and NaN (otherwise).
  Subnormals m/4 * 2^-14.

Encoding a float32 value v (readings where the pages are silent are marked R):

* round to the nearest representable value, ties to the even code (the
  accumulation-precision example on the course page -- "promoting every 8
  terms gives exactly 300" -- holds with ties-to-even and fails with ties-away);
* saturate: any |v| above the largest finite value becomes +-fmax (the lesson's
  worked example: a spike of 300 at scale 448/240 "clips at 448");
* R: +-inf saturates to +-fmax as well;
* R: NaN encodes to sign | 0x7F (a NaN code in both formats);
* R: the sign of zero is kept (-0 and negative underflow give 0x80);
* R: subnormal FP8 values are produced (gradual underflow).

bf16: 8 significant bits, round to nearest even (the course page's precision
paragraph: 257 rounds to 256, not 258).  Overflow follows IEEE round-to-nearest
(values at or beyond max + half an ulp become inf).  NaN stays NaN.

e8m0 (the shared scale of the 32-element MX groups named on the course page's
absmax paragraph): an 8-bit biased exponent, value 2^(code - 127); code 255 is
NaN.

Everything here is vectorised NumPy in float64 (all FP8 / bf16 / fp32 values
are exact in float64).  ``encode_scalar`` / ``decode_scalar`` are independent
pure-Python versions over ``fractions.Fraction`` used to cross-check the
vectorised ones.
"""

from __future__ import annotations

import bisect
import math
from fractions import Fraction

import numpy as np

E4M3 = 0
E5M2 = 1

# (exponent bits, mantissa bits, bias, largest finite value)
_SPEC = {
    E4M3: (4, 3, 7, 448.0),
    E5M2: (5, 2, 15, 57344.0),
}

FMAX = {E4M3: 448.0, E5M2: 57344.0}


def fmt_name(fmt: int) -> str:
    return {E4M3: "E4M3", E5M2: "E5M2"}[fmt]


# --------------------------------------------------------------------------- decode


def decode(codes, fmt: int) -> np.ndarray:
    """FP8 codes (uint8 array) -> float64 values, from the closed form."""
    ebits, mbits, bias, _ = _SPEC[fmt]
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = c & ((1 << mbits) - 1)
    sign = np.where(s == 1, -1.0, 1.0)
    sub = m.astype(np.float64) / (1 << mbits) * 2.0 ** (1 - bias)
    nrm = (1.0 + m.astype(np.float64) / (1 << mbits)) * np.exp2((e - bias).astype(np.float64))
    val = sign * np.where(e == 0, sub, nrm)
    emax_field = (1 << ebits) - 1
    if fmt == E4M3:
        nan = (e == emax_field) & (m == (1 << mbits) - 1)
        val = np.where(nan, np.nan, val)
    else:
        top = e == emax_field
        val = np.where(top & (m == 0), sign * np.inf, val)
        val = np.where(top & (m != 0), np.nan, val)
    return val


def decode_scalar(code: int, fmt: int) -> float:
    """Pure-Python decode of one code (independent of :func:`decode`)."""
    ebits, mbits, bias, _ = _SPEC[fmt]
    s = code >> 7
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if fmt == E4M3 and e == 15 and m == 7:
        return math.nan
    if fmt == E5M2 and e == 31:
        return math.nan if m else (-math.inf if s else math.inf)
    if e == 0:
        mag = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return float(-mag if s else mag)


def positive_grid(fmt: int):
    """(codes, values) of the non-negative finite codes, ascending (0x00 .. fmax)."""
    codes = np.arange(128, dtype=np.uint8)
    vals = decode(codes, fmt)
    keep = np.isfinite(vals)
    return codes[keep], vals[keep]


# --------------------------------------------------------------------------- encode


def encode(v, fmt: int) -> np.ndarray:
    """float32 values -> FP8 codes: nearest value, ties to even code, saturating.

    ``v`` is converted to float32 first (the product the kernels round).  The
    search is over the explicit table of finite FP8 values: the lower and upper
    neighbours of |v| are found and the midpoint decides.
    """
    x = np.asarray(v, dtype=np.float32)
    codes, vals = positive_grid(fmt)
    fmax = vals[-1]
    with np.errstate(invalid="ignore"):
        a = np.abs(x.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, fmax))  # saturation (inf included)
    lo = np.searchsorted(vals, a, side="right") - 1  # vals[lo] <= a
    hi = np.minimum(lo + 1, len(vals) - 1)
    mid = (vals[lo] + vals[hi]) * 0.5  # exact in float64
    up = (a > mid) | ((a == mid) & (codes[hi] % 2 == 0) & (hi != lo))
    mag = np.where(up, codes[hi], codes[lo]).astype(np.uint8)
    mag = np.where(nan, np.uint8(0x7F), mag)
    sign = np.signbit(x).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


_SCALAR_GRID = {}


def _scalar_grid(fmt: int):
    if fmt not in _SCALAR_GRID:
        pairs = []
        for c in range(128):
            d = decode_scalar(c, fmt)
            if math.isfinite(d):
                pairs.append((Fraction(d), c))
        pairs.sort()
        _SCALAR_GRID[fmt] = ([p[0] for p in pairs], [p[1] for p in pairs])
    return _SCALAR_GRID[fmt]


def encode_scalar(v: float, fmt: int) -> int:
    """Pure-Python encode of one float32 value over exact rationals."""
    v = float(np.float32(v))
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    if math.isnan(v):
        return sign | 0x7F
    vals, codes = _scalar_grid(fmt)
    if math.isinf(v):
        return sign | codes[-1]
    a = abs(Fraction(v))
    if a >= vals[-1]:
        return sign | codes[-1]
    i = bisect.bisect_right(vals, a) - 1
    lo, hi = vals[i], vals[i + 1]
    if a - lo < hi - a:
        c = codes[i]
    elif a - lo > hi - a:
        c = codes[i + 1]
    else:
        c = codes[i] if codes[i] % 2 == 0 else codes[i + 1]
    return sign | c


# --------------------------------------------------------------------------- bf16


def bf16_round_bits(v) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest even.

    For each value the two bf16 neighbours around it (truncation toward zero and
    the next value up in magnitude) are compared to |v| exactly in float64; the
    midpoint goes to the neighbour whose last kept bit is 0.
    """
    x = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    sign = u & 0x80000000
    mag = u & 0x7FFFFFFF
    lower = mag & 0x7FFF0000
    upper = lower + 0x10000
    with np.errstate(invalid="ignore"):
        lo_val = lower.astype(np.uint32).view(np.float32).astype(np.float64)
    up_bits = np.minimum(upper, 0x7F800000).astype(np.uint32)
    up_val = up_bits.view(np.float32).astype(np.float64)
    # past the largest finite bf16 the next "value" for rounding is 2^128
    up_val = np.where(lower == 0x7F7F0000, 2.0 ** 128, up_val)
    with np.errstate(invalid="ignore"):
        a = np.abs(x.astype(np.float64))
    mid = (lo_val + up_val) * 0.5
    lower_even = ((lower >> 16) & 1) == 0
    take_up = (a > mid) | ((a == mid) & ~lower_even)
    res = np.where(take_up, upper, lower)
    res = np.minimum(res, 0x7F800000)  # overflow -> inf
    isnan = np.isnan(x)
    res = np.where(isnan, (mag >> 16 << 16) | 0x00400000, res)
    res = np.where(np.isinf(x), 0x7F800000, res)
    out = ((res | sign) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def to_bf16(v) -> np.ndarray:
    """float32 values rounded to bf16 (RNE), returned as float32 arrays."""
    return bf16_bits_to_f32(bf16_round_bits(v))


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^(floor(log2|x|) - 7)), min-normal spacing at 0."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    e = np.maximum(e, -126.0)
    return np.exp2(e - 7.0)


# --------------------------------------------------------------------------- e8m0


def e8m0_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2((c - 127).astype(np.float64)))
