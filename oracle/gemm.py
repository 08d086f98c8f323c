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
* G[m, n] = sum_g alpha_g beta_g (max_{k in g} 2^ea_k)(max_{k in g} 2^eb_k) over
  the aligned groups g of 8 consecutive k, where ea / eb is the binade exponent
  of the FP8 code (exponent field minus bias; the minimum normal exponent for
  subnormals and zeros) and alpha_g / beta_g the group's dequantisation factors.
  Since |a| < 2^(ea+1) for every code, 4 G bounds sum_g max_{k in g} |a_k b_k|.
  The tests use G to bound the error of an accumulator that sums each run of 8
  products in a fixed-point window below its largest exponent sum before
  promoting the run to fp32 (the course page's "about 14 bits", measured on the
  matrix cores this path runs on).

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


def code_binade(q, fmt) -> np.ndarray:
    """2^e for each FP8 code: e = exponent field - bias (1 - bias for subnormals and zero)."""
    mbits, bias = (3, 7) if fmt == fp8.E4M3 else (2, 15)
    ef = (np.asarray(q, dtype=np.uint8).astype(np.int64) & 0x7F) >> mbits
    return np.exp2((np.maximum(ef, 1) - bias).astype(np.float64))


def group_exponent_bound(q, fmt, gran, scale_inv, group: int = 8) -> np.ndarray:
    """[rows][K/group]: max over each run of 2^e(code), times the run's dequantisation factor."""
    rows, k = np.asarray(q).shape
    e = code_binade(q, fmt).reshape(rows, k // group, group).max(axis=2)
    ones = np.ones((rows, k), dtype=np.uint8) * 0x38  # 1.0 in E4M3: picks out the factors
    f = dequant(ones, fp8.E4M3, gran, scale_inv)[:, ::group]
    return e * f


def gemm_ref(A, fmt_a, sa, gran_a, B, fmt_b, sb, gran_b, rows=None, cols=None):
    """(C, S, G) in float64 for C = A . B^T; optional row / column subsets of the output."""
    A = np.asarray(A, dtype=np.uint8)
    B = np.asarray(B, dtype=np.uint8)
    Ad = dequant(A, fmt_a, gran_a, sa)
    Bd = dequant(B, fmt_b, gran_b, sb)
    Ae = group_exponent_bound(A, fmt_a, gran_a, sa)
    Be = group_exponent_bound(B, fmt_b, gran_b, sb)
    if rows is not None:
        Ad, Ae = Ad[rows], Ae[rows]
    if cols is not None:
        Bd, Be = Bd[cols], Be[cols]
    C = Ad @ Bd.T
    S = np.abs(Ad) @ np.abs(Bd).T
    G = Ae @ Be.T
    return C, S, G


def to_bf16(c) -> np.ndarray:
    """float32 GEMM output -> bf16 (returned as float32 values)."""
    return fp8.to_bf16(np.asarray(c, dtype=np.float32))
