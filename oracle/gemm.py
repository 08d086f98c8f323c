"""FP8 x FP8 GEMM reference: fp64 sum over dequantised operands, plus bound matrices.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The layer computes ``C = A . B^T`` (``Y = X W^T``, the nn.Linear convention the
Transformer Engine tutorial uses) from FP8 operands A [M][K] and B [N][K] and
their scales ("Week 14" course page, FP8 bullet: matmuls run in FP8;
accumulation-precision bullet: products are summed in a wider accumulator and
partial sums are promoted to fp32).  The definition, written out:

    C[m, n] = sum_k  dec(A[m, k]) * alpha(m, k) * dec(B[n, k]) * beta(n, k)

where alpha / beta are the dequantisation factors of the operand's granularity:

* per tensor: the tensor's scale_inv (a float32 scalar);
* 1x128 tile (A): scale_inv[k // 128][m];
* 128x128 block (B): scale_inv[n // 128][k // 128];
* MX 1x32: 2^(code[row][k // 32] - 127).

The sum is taken in float64 (``numpy`` matmul); every FP8 product and every
power-of-two or float32 factor is exact there, so the only rounding is float64
summation, far below any tolerance used.

Two non-negative bound matrices come with it:

* S[m, n] = sum_k |a_k b_k|  (the sum of product magnitudes, dequantised);
* G[m, n] = sum_g (max_{k in g} |a_k|)(max_{k in g} |b_k|) over the aligned
  groups g of 8 consecutive k -- an upper bound of sum_g max_{k in g} |a_k b_k|,
  used by the tests to bound the error of an accumulator that sums short runs
  of products at reduced precision before promoting them to fp32.

A bf16 output is the float32 result rounded to nearest even (``oracle.fp8``).
"""

from __future__ import annotations

import numpy as np

from . import fp8

TENSOR, TILE_1x128, BLOCK_128x128, MX_1x32 = 0, 1, 2, 3


def dequant(q, fmt, gran, scale_inv) -> np.ndarray:
    """FP8 codes [rows][K] -> float64 values times their dequantisation factors."""
    q = np.asarray(q, dtype=np.uint8)
    rows, k = q.shape
    v = fp8.decode(q, fmt)
    if gran == TENSOR:
        f = np.float64(np.float32(scale_inv))
        return v * f
    if gran == TILE_1x128:
        s = np.asarray(scale_inv, dtype=np.float32).astype(np.float64)  # [K/128][rows]
        assert s.shape == (k // 128, rows)
        return v * np.repeat(s.T, 128, axis=1)
    if gran == BLOCK_128x128:
        s = np.asarray(scale_inv, dtype=np.float32).astype(np.float64)  # [ceil(rows/128)][K/128]
        assert s.shape == (-(-rows // 128), k // 128)
        full = np.repeat(np.repeat(s, 128, axis=0)[:rows], 128, axis=1)
        return v * full
    if gran == MX_1x32:
        c = np.asarray(scale_inv, dtype=np.uint8)  # [rows][K/32]
        assert c.shape == (rows, k // 32)
        f = fp8.e8m0_decode(c)
        return v * np.repeat(f, 32, axis=1)
    raise ValueError("granularity")


def group_max(v, group: int = 8) -> np.ndarray:
    """max |v| over aligned runs of ``group`` columns -> [rows][K/group]."""
    a = np.abs(v)
    rows, k = a.shape
    return a.reshape(rows, k // group, group).max(axis=2)


def gemm_ref(A, fmt_a, sa, gran_a, B, fmt_b, sb, gran_b, rows=None, cols=None):
    """(C, S, G) in float64 for C = A . B^T; optional row / column subsets of the output."""
    Ad = dequant(A, fmt_a, gran_a, sa)
    Bd = dequant(B, fmt_b, gran_b, sb)
    if rows is not None:
        Ad = Ad[rows]
    if cols is not None:
        Bd = Bd[cols]
    C = Ad @ Bd.T
    S = np.abs(Ad) @ np.abs(Bd).T
    G = group_max(Ad) @ group_max(Bd).T
    return C, S, G


def to_bf16(c) -> np.ndarray:
    """float32 GEMM output -> bf16 (returned as float32 values)."""
    return fp8.to_bf16(np.asarray(c, dtype=np.float32))
