"""Pins of the oracle's quantizers' layouts, GEMM reference, accumulation example and int8 absmax (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from conftest import read_golden
from oracle import absmax, accum, fp8, gemm, quantize, recipe

E4M3, E5M2 = fp8.E4M3, fp8.E5M2
f32 = np.float32


# --------------------------------------------------------------------------- accumulation example


def test_accumulation_example_from_pages():
    rows = read_golden("e4m3_accumulation.txt")
    for name, term, count, interval, expected, steps in rows:
        term, count, interval, expected = float(term), int(count), int(interval), float(expected)
        if name == "single_add":
            v = float(fp8.decode(fp8.encode(f32(64.0 + term), E4M3), E4M3))
            assert v == expected
        elif name == "naive":
            total, trace = accum.fp8_running_sum([term] * count, E4M3, trace=True)
            assert total == expected
            first = trace.index(expected) + 1
            assert first == int(steps.split()[0])
            assert all(v == expected for v in trace[first - 1:])
        elif name == "promoted":
            assert accum.promoted_sum([term] * count, interval, E4M3) == expected


def test_promotion_pins_ties_to_even():
    """With ties-away the promoted sum would be 324: 21 -> 22 and 25 -> 26 inside each run of 8."""
    assert float(fp8.decode(fp8.encode(f32(21.0), E4M3), E4M3)) == 20.0
    assert float(fp8.decode(fp8.encode(f32(23.0), E4M3), E4M3)) == 24.0
    run = accum.fp8_running_sum([3.0] * 8, E4M3)
    assert run == 24.0


# --------------------------------------------------------------------------- int8 absmax


def test_absmax_int8_example_from_pages():
    for name, xs, qs, deq in read_golden("absmax_int8.txt"):
        x = np.array([float(v) for v in xs.split()])
        if name == "block2":
            q, steps = absmax.absmax_quantize_blocks(x, 2)
            want = [int(v) for v in qs.split() if v != "*"]
            assert list(q[:2]) == want
            continue
        q, step, back = absmax.absmax_quantize(x)
        assert list(q) == [int(v) for v in qs.split()]
        if deq != "-":
            assert np.allclose(np.round(back, 3), [float(v) for v in deq.split()])
        if name == "outlier":
            # all numbers up to 0.5 in magnitude get 5 levels (-2 .. 2)
            grid = np.arange(-0.5, 0.5001, 0.001)
            levels = np.unique(np.rint(grid / step))
            assert len(levels) == 5


# --------------------------------------------------------------------------- quantizer layouts


def test_fp32_product_then_encode_is_the_definition():
    """The product is rounded to float32 before the FP8 encode (double rounding, by definition).

    Searches inputs whose float32 product lands exactly on a midpoint between two
    E4M3 values while the exact product lies on the odd side: the float32 path
    goes to the even code, rounding the exact product directly would not.
    """
    codes, vals = fp8.positive_grid(E4M3)
    rng = np.random.default_rng(14)
    found = 0
    for s in rng.uniform(1.0, 2.0, 64).astype(np.float32):
        for i in range(40, len(vals) - 1):
            mid = f32((vals[i] + vals[i + 1]) / 2)
            x = f32(mid / s)
            for _ in range(6):
                if f32(x * s) == mid and float(x) * float(s) != float(mid):
                    q, _ = quantize.quantize_tensor(np.array([x], np.float32), s, E4M3)
                    even = codes[i] if codes[i] % 2 == 0 else codes[i + 1]
                    assert q[0] == even
                    exact_side = codes[i + 1] if float(x) * float(s) > float(mid) else codes[i]
                    found += int(exact_side != even)
                x = np.nextafter(x, f32(np.inf))
    assert found > 0


def test_cast_transpose_is_transpose():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((37, 70)).astype(np.float32)
    q, qT, a = quantize.cast_transpose(x, f32(30.0), E5M2)
    assert np.array_equal(qT, q.T) and a == recipe.amax(x)
    q2, _ = quantize.quantize_tensor(x, f32(30.0), E5M2)
    assert np.array_equal(q, q2)


def test_tile_scale_layout_brute_force():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((5, 384)) * np.exp2(rng.integers(-4, 4, (5, 384)))).astype(np.float32)
    q, sinv = quantize.quantize_tile_1x128(x, E4M3)
    for m in range(5):
        for kb in range(3):
            tile = x[m, kb * 128:(kb + 1) * 128]
            a = np.abs(tile).max()
            s = f32(448.0) / f32(a)
            assert sinv[kb, m] == f32(1.0) / s
            for k in range(0, 128, 17):
                assert q[m, kb * 128 + k] == fp8.encode_scalar(float(f32(tile[k] * s)), E4M3)


def test_block_scale_layout_ragged_rows():
    rng = np.random.default_rng(9)
    w = rng.standard_normal((200, 256)).astype(np.float32)
    q, sinv = quantize.quantize_block_128x128(w, E4M3)
    assert sinv.shape == (2, 2)
    a = np.abs(w[128:200, 128:256]).max()
    assert sinv[1, 1] == f32(1) / (f32(448) / f32(a))


# --------------------------------------------------------------------------- GEMM reference


def _codes(rng, shape, fmt):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    bad = ~np.isfinite(fp8.decode(c, fmt))
    c[bad] = 0x38 if fmt == E4M3 else 0x3C
    return c


def test_hundred_threes_gemm_is_300():
    """Course page: 100 threes promoted to fp32 give exactly 300 (A = 3.0 x 100 + 28 zeros, B = 1.0)."""
    A = np.zeros((1, 128), np.uint8)
    A[0, :100] = 0x44
    B = np.full((1, 128), 0x38, np.uint8)
    C, S, G = gemm.gemm_ref(A, E4M3, f32(1), gemm.TENSOR, B, E4M3, f32(1), gemm.TENSOR)
    # G: 13 runs holding threes (2^1 * 2^0 each) + 3 runs of zero codes (2^-6 * 2^0 each)
    assert C[0, 0] == 300.0 and S[0, 0] == 300.0 and G[0, 0] == 13 * 2.0 + 3 * 2.0 ** -6


def test_gemm_closed_forms():
    eye = np.zeros((128, 128), np.uint8)
    np.fill_diagonal(eye, 0x38)
    rng = np.random.default_rng(10)
    B = _codes(rng, (64, 128), E5M2)
    C, _, _ = gemm.gemm_ref(eye, E4M3, f32(0.5), gemm.TENSOR, B, E5M2, f32(4.0), gemm.TENSOR)
    assert np.array_equal(C, 2.0 * fp8.decode(B, E5M2).T)
    ones = np.full((3, 256), 0x38, np.uint8)
    C, S, _ = gemm.gemm_ref(ones, E4M3, f32(1), gemm.TENSOR, ones, E4M3, f32(1), gemm.TENSOR)
    assert np.all(C == 256.0) and np.all(S == 256.0)


@pytest.mark.parametrize("mode", ["tensor", "blockwise", "tile2", "mx"])
def test_gemm_brute_force_fractions(mode):
    rng = np.random.default_rng(11)
    M, N, K = 3, 5, 256
    fa, fb = (E5M2, E4M3) if mode == "tensor" else (E4M3, E4M3)
    A, B = _codes(rng, (M, K), fa), _codes(rng, (N, K), fb)
    if mode == "tensor":
        sa, sb, ga, gb = f32(0.37), f32(1.0 / 3.0), gemm.TENSOR, gemm.TENSOR
        fa_ = lambda m, k: Fraction(float(sa))
        fb_ = lambda n, k: Fraction(float(sb))
    elif mode == "blockwise":
        sa = rng.uniform(0.1, 3, (K // 128, M)).astype(np.float32)
        sb = rng.uniform(0.1, 3, (1, K // 128)).astype(np.float32)
        ga, gb = gemm.TILE_1x128, gemm.BLOCK_128x128
        fa_ = lambda m, k: Fraction(float(sa[k // 128, m]))
        fb_ = lambda n, k: Fraction(float(sb[n // 128, k // 128]))
    elif mode == "tile2":
        sa = rng.uniform(0.1, 3, (K // 128, M)).astype(np.float32)
        sb = rng.uniform(0.1, 3, (K // 128, N)).astype(np.float32)
        ga, gb = gemm.TILE_1x128, gemm.TILE_1x128
        fa_ = lambda m, k: Fraction(float(sa[k // 128, m]))
        fb_ = lambda n, k: Fraction(float(sb[k // 128, n]))
    else:
        sa = rng.integers(100, 150, (M, K // 32)).astype(np.uint8)
        sb = rng.integers(100, 150, (N, K // 32)).astype(np.uint8)
        ga, gb = gemm.MX_1x32, gemm.MX_1x32
        fa_ = lambda m, k: Fraction(2) ** (int(sa[m, k // 32]) - 127)
        fb_ = lambda n, k: Fraction(2) ** (int(sb[n, k // 32]) - 127)
    C, S, G = gemm.gemm_ref(A, fa, sa, ga, B, fb, sb, gb)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            smag = Fraction(0)
            for k in range(K):
                p = (Fraction(fp8.decode_scalar(int(A[m, k]), fa)) * fa_(m, k) *
                     Fraction(fp8.decode_scalar(int(B[n, k]), fb)) * fb_(n, k))
                exact += p
                smag += abs(p)
            assert abs(Fraction(C[m, n]) - exact) <= smag * Fraction(1, 2 ** 50)
            assert abs(Fraction(S[m, n]) - smag) <= smag * Fraction(1, 2 ** 50)


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3)])
def test_group_exponent_bound_brackets_group_products(fa, fb):
    """4 G >= sum over runs of 8 of the largest |product|; G <= sum of max|a| max|b| (normal codes)."""
    rng = np.random.default_rng(12)
    A, B = _codes(rng, (4, 128), fa), _codes(rng, (6, 128), fb)
    sa, sb = f32(0.75), f32(3.0)
    C, S, G = gemm.gemm_ref(A, fa, sa, gemm.TENSOR, B, fb, sb, gemm.TENSOR)
    a, b = fp8.decode(A, fa) * float(sa), fp8.decode(B, fb) * float(sb)
    for m in range(4):
        for n in range(6):
            p = np.abs(a[m] * b[n]).reshape(16, 8)
            assert 4 * G[m, n] >= p.max(axis=1).sum() and S[m, n] >= abs(C[m, n])
    # exact binades of normal codes: G equals the brute-force sum of run maxima of 2^e
    An = np.full((1, 128), 0x38, np.uint8)
    An[0, 5] = 0x50  # 2^3 in E4M3
    Bn = np.full((1, 128), 0x40, np.uint8)  # 2.0
    _, _, G1 = gemm.gemm_ref(An, E4M3, f32(1), gemm.TENSOR, Bn, E4M3, f32(1), gemm.TENSOR)
    assert G1[0, 0] == 8 * 2 + 15 * 2


def test_gemm_subset_rows_cols():
    rng = np.random.default_rng(13)
    A, B = _codes(rng, (20, 128), E4M3), _codes(rng, (30, 128), E4M3)
    C, S, G = gemm.gemm_ref(A, E4M3, f32(2), gemm.TENSOR, B, E4M3, f32(3), gemm.TENSOR)
    r, c = np.array([1, 7, 19]), np.array([0, 29])
    C2, S2, G2 = gemm.gemm_ref(A, E4M3, f32(2), gemm.TENSOR, B, E4M3, f32(3), gemm.TENSOR, rows=r, cols=c)
    assert np.array_equal(C2, C[np.ix_(r, c)]) and np.array_equal(G2, G[np.ix_(r, c)])


def test_bf16_output_rounding():
    assert gemm.to_bf16(np.array([257.0, 259.0, -257.0], np.float32)).tolist() == [256.0, 260.0, -256.0]
