"""Quantizers: per-tensor (delayed), 1x128 tiles, 128x128 blocks, MX 1x32; cast-transpose.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Every quantizer computes ``q = enc_F(fp32(x * s))``: one float32 multiply
rounded to nearest even, then the saturating FP8 encode of ``oracle.fp8``.  The
double rounding (float32 product, then FP8) is part of the definition: it is
what a float32 pipeline computes.  bf16 inputs are exact in float32.

Granularities ("Week 14" course page, absmax paragraph: a scale per tensor, per
channel or per block; MX gives every 32 numbers a shared scale; DeepSeek-V3
used a scale for every 128 activation values and every 128 x 128 weight block):

* per tensor: the caller's delayed scale (``oracle.recipe``); returns the
  tensor's amax to be recorded in the history;
* 1x128 tiles along the contraction (column) axis of a row-major [rows][cols]
  activation: scale_inv stored [cols/128][rows] (tile-column major);
* 128x128 blocks of a row-major [rows][cols] weight: scale_inv stored
  [ceil(rows/128)][cols/128]; a last, partial row-block uses the rows present;
* MX 1x32 groups along the column axis: e8m0 codes stored [rows][cols/32];
  the elements are multiplied by 2^-E (exact) before the encode.

Cast-transpose returns the same bytes as the per-tensor quantizer and their
transpose: qT[c][r] = q[r][c].

Blockwise cast-transpose (the blockwise recipe's backward operands): the
transposed copy carries the scales of its own contraction axis, which is the
source's row axis.  For 1x128 tiles, the copy of x^T is quantised in runs of
128 consecutive source rows of one column (a 128x1 run of x, a 1x128 run of
x^T); for 128x128 blocks the block, and so its scale, is the same either way
round, so the copy is the transpose of the codes and of the scale matrix.
"""

from __future__ import annotations

import numpy as np

from . import fp8, recipe


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def scaled_encode(x, s, fmt) -> np.ndarray:
    """enc(fp32(x * s)) with ``s`` broadcast against ``x``."""
    with np.errstate(over="ignore", invalid="ignore"):
        v = (_f32(x) * np.asarray(s, dtype=np.float32)).astype(np.float32)
    return fp8.encode(v, fmt)


def quantize_tensor(x, scale, fmt):
    """Per-tensor quantisation with a given (delayed) scale -> (q, amax)."""
    x = _f32(x)
    return scaled_encode(x, np.float32(scale), fmt), recipe.amax(x)


def quantize_tile_1x128(x, fmt):
    """1x128 tiles along columns -> (q [rows][cols], scale_inv [cols/128][rows])."""
    x = _f32(x)
    rows, cols = x.shape
    assert cols % 128 == 0
    t = x.reshape(rows, cols // 128, 128)
    with np.errstate(invalid="ignore"):
        a = np.abs(t).max(axis=2)  # [rows][cols/128], NaN-propagating
    s, s_inv = recipe.current_scale(a, fmt)
    q = scaled_encode(t, s[:, :, None], fmt).reshape(rows, cols)
    return q, np.ascontiguousarray(s_inv.T)


def quantize_block_128x128(w, fmt):
    """128x128 blocks -> (q [rows][cols], scale_inv [ceil(rows/128)][cols/128])."""
    w = _f32(w)
    rows, cols = w.shape
    assert cols % 128 == 0
    nrb, ncb = -(-rows // 128), cols // 128
    a = np.zeros((nrb, ncb), dtype=np.float32)
    for i in range(nrb):
        blk = w[i * 128:(i + 1) * 128].reshape(-1, ncb, 128)
        with np.errstate(invalid="ignore"):
            a[i] = np.abs(blk).max(axis=(0, 2))
    s, s_inv = recipe.current_scale(a, fmt)
    s_full = np.repeat(np.repeat(s, 128, axis=0)[:rows], 128, axis=1)
    return scaled_encode(w, s_full, fmt), s_inv


def quantize_mx_1x32(x, fmt):
    """MX groups of 32 along columns -> (q [rows][cols], e8m0 [rows][cols/32])."""
    x = _f32(x)
    rows, cols = x.shape
    assert cols % 32 == 0
    g = x.reshape(rows, cols // 32, 32)
    with np.errstate(invalid="ignore"):
        a = np.abs(g).max(axis=2)
    codes = recipe.mx_exponent(a, fmt)
    e = codes.astype(np.int64) - 127
    # 2^-E as float32 (exact for |E| <= 126; 2^127 also exact); NaN groups use 1
    mult = np.where(codes == 255, 1.0, np.exp2(-e.astype(np.float64))).astype(np.float32)
    q = scaled_encode(g, mult[:, :, None], fmt).reshape(rows, cols)
    return q, codes


def cast_transpose(x, scale, fmt):
    """Per-tensor quantisation plus the transposed bytes -> (q, qT, amax)."""
    q, a = quantize_tensor(x, scale, fmt)
    return q, np.ascontiguousarray(q.T), a


def quantize_tile_128x1(x, fmt):
    """128x1 runs down the columns (128 consecutive rows of one column) ->
    (q [rows][cols], scale_inv [rows/128][cols])."""
    x = _f32(x)
    rows, cols = x.shape
    assert rows % 128 == 0
    t = x.reshape(rows // 128, 128, cols)
    with np.errstate(invalid="ignore"):
        a = np.abs(t).max(axis=1)  # [rows/128][cols], NaN-propagating
    s, s_inv = recipe.current_scale(a, fmt)
    q = scaled_encode(t, s[:, None, :], fmt).reshape(rows, cols)
    return q, s_inv


def cast_transpose_blockwise(x, fmt, granularity):
    """(q, q_scale_inv, qT, qT_scale_inv) for granularity 1 (TILE_1x128) or 2 (BLOCK_128x128).

    TILE_1x128: q in 1x128 runs along the columns (scale_inv [cols/128][rows]); qT = the
    transposed codes of x quantised in 128x1 runs (scale_inv [rows/128][cols]).
    BLOCK_128x128: q in 128x128 blocks; qT and its scale_inv are the transposes.
    """
    if granularity == 1:
        q, q_sinv = quantize_tile_1x128(x, fmt)
        qc, qt_sinv = quantize_tile_128x1(x, fmt)
        return q, q_sinv, np.ascontiguousarray(qc.T), qt_sinv
    if granularity == 2:
        q, q_sinv = quantize_block_128x128(x, fmt)
        return q, q_sinv, np.ascontiguousarray(q.T), np.ascontiguousarray(q_sinv.T)
    raise ValueError("granularity")


def cast_diagnostics(x, scale, fmt):
    """(saturated, underflowed, nan) element counts of the per-tensor cast with ``scale``:
    saturated = |fp32(x * s)| > fmax (the code is clipped), underflowed = x finite and
    non-zero whose code decodes to 0, nan = NaN inputs."""
    x = _f32(x)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (x * np.float32(scale)).astype(np.float32)
        saturated = int(np.count_nonzero(np.abs(y) > fp8.FMAX[fmt]))
    q = fp8.encode(y, fmt)
    finite_nz = np.isfinite(x) & (x != 0)
    underflowed = int(np.count_nonzero(finite_nz & (fp8.decode(q, fmt) == 0)))
    return saturated, underflowed, int(np.count_nonzero(np.isnan(x)))
