"""GPU parity of fp8_gemm against the fp64 oracle, within the bound derived from the
matrix cores' accumulation (see gpu_util.gemm_bound); exact pins where the result is exact."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import DEV, announce, check_gemm, np_of  # noqa: E402
from oracle import fp8 as ofp8, gemm as og, quantize as oq  # noqa: E402


@pytest.fixture(scope="module")
def sq():
    import scaled_quantize_gemm_amd as m

    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _codes(rng, shape, fmt, realistic=True):
    """FP8 codes: quantised Gaussian data (realistic) or uniform over all finite codes."""
    if realistic:
        x = rng.standard_normal(shape).astype(np.float32)
        return oq.quantize_tensor(x, np.float32(ofp8.FMAX[fmt] / np.abs(x).max()), fmt)[0]
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[~np.isfinite(ofp8.decode(c, fmt))] = 0
    return c


def _scal(v):
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def test_hundred_threes_is_exactly_300(sq):
    """Course page accumulation example as a GEMM: fp32 promotion gives exactly 300 (not 64)."""
    announce("100 threes")
    A = np.zeros((1, 128), np.uint8)
    A[0, :100] = 0x44  # 3.0
    B = np.full((1, 128), 0x38, np.uint8)  # 1.0
    C = sq.fp8_gemm(_t(A), 0, _scal(1.0), 0, _t(B), 0, _scal(1.0), 0, sq.OUT_F32)
    torch.cuda.synchronize()
    assert np_of(C)[0, 0] == 300.0


def test_bf16_epilogue_rounds_to_nearest_even(sq):
    """Course page precision paragraph: 257 -> 256 in bf16 (ties to even); 259 -> 260."""
    announce("bf16 epilogue 257")
    A = np.zeros((4, 128), np.uint8)
    B = np.zeros((1, 128), np.uint8)
    B[0, :] = 0x38  # 1.0
    # row sums: 256 + 1 = 257, 256 + 3 = 259, -(256 + 1), 255
    A[0, 0], A[0, 8] = 0x78, 0x38  # 256 in E4M3 = 0x78, then 1.0 in another run of 8
    A[1, 0], A[1, 8] = 0x78, 0x44  # 256 + 3
    A[2, 0], A[2, 8] = 0xF8, 0xB8  # -256 - 1
    A[3, 0], A[3, 8] = 0x78, 0xB8  # 256 - 1 = 255
    C = sq.fp8_gemm(_t(A), 0, _scal(1.0), 0, _t(B), 0, _scal(1.0), 0, sq.OUT_BF16)
    torch.cuda.synchronize()
    assert np_of(C)[:, 0].tolist() == [256.0, 260.0, -256.0, 255.0]


def test_accumulator_runs_of_eight(sq):
    """The matrix-core behaviour the tolerance relies on: a small product in the same run of 8
    as a large one keeps only bits down to 2^(E-13) (E = the run's largest operand-exponent
    sum); in another run it is added in fp32."""
    announce("accumulator model")
    A = np.zeros((2, 128), np.uint8)
    B = np.zeros((1, 128), np.uint8)
    B[0, :] = 0x7E  # 448
    A[:, 0] = 0x7E  # 448 * 448 = 200704 (exponent sum 16)
    A[0, 1] = 0x20  # 2^-3 * 448 = 56 -> same run: bits below 2^3 truncated -> 56 kept
    A[1, 9] = 0x20  # other run -> exact in fp32
    A[0, 2] = 0x01  # 2^-9 * 448 = 0.875 -> same run -> lost
    A[1, 10] = 0x01  # other run -> kept (fp32 spacing at 2^17 is 2^-6)
    C = np_of(sq.fp8_gemm(_t(A), 0, _scal(1.0), 0, _t(B), 0, _scal(1.0), 0, sq.OUT_F32))[:, 0]
    torch.cuda.synchronize()
    assert C[0] == 200704.0 + 56.0
    assert C[1] == 200704.0 + 56.0 + 0.875
    Cr, S, G = og.gemm_ref(A, 0, np.float32(1), og.TENSOR, B, 0, np.float32(1), og.TENSOR)
    check_gemm(C[:, None], Cr, S, G, 128, "tensor", False, "accumulator model")


def test_k_zero_gives_zero(sq):
    announce("K = 0")
    A = torch.empty((5, 0), dtype=torch.uint8, device=DEV)
    B = torch.empty((7, 0), dtype=torch.uint8, device=DEV)
    C = sq.fp8_gemm(A, 0, _scal(2.0), 0, B, 0, _scal(3.0), 0, sq.OUT_F32)
    torch.cuda.synchronize()
    assert np.all(np_of(C) == 0)


TENSOR_CASES = [(256, 256, 256), (200, 300, 384), (1, 1, 128), (130, 70, 128), (33, 517, 256), (512, 384, 1024)]


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1)])
@pytest.mark.parametrize("out", [0, 1])
@pytest.mark.parametrize("mnk", TENSOR_CASES)
def test_tensor_scaled_gemm(sq, fa, fb, out, mnk):
    M, N, K = mnk
    announce("tensor gemm", fa, fb, out, mnk)
    rng = np.random.default_rng(M * 7 + N * 3 + K + fa * 5 + fb * 11)
    for realistic in (True, False):
        A, B = _codes(rng, (M, K), fa, realistic), _codes(rng, (N, K), fb, realistic)
        sa, sb = np.float32(rng.uniform(0.001, 0.1)), np.float32(rng.uniform(0.001, 0.1))
        C = sq.fp8_gemm(_t(A), fa, _scal(sa), 0, _t(B), fb, _scal(sb), 0, out)
        torch.cuda.synchronize()
        Cr, S, G = og.gemm_ref(A, fa, sa, og.TENSOR, B, fb, sb, og.TENSOR)
        check_gemm(np_of(C), Cr, S, G, K, "tensor", out == 1, f"tensor {mnk} {fa}{fb} out{out} real={realistic}")


# per-tensor problems below 128 tiles of 256 x 128 run on 256 x 64 tiles, from 128 tiles on on
# 256 x 128 tiles, 128 x 64 tiles where at most 256 of them cover C (and from 256 tiles of
# 256 x 256 on the 256 x 256 kernel): both sides of each
# boundary, with ragged last tiles, against the oracle on sampled rows
@pytest.mark.parametrize("mnk", [
    (256, 127 * 128, 256),       # 127 tiles of 256 x 128: 256 x 64 tiles
    (256, 128 * 128, 256),       # 128: 256 x 128 tiles
    (2 * 256 - 5, 8024, 384),    # 2 x 63 = 126, ragged M and N: 256 x 64 tiles
    (2 * 256, 64 * 128, 128),    # 2 x 64 = 128: 256 x 128 tiles
    (3840, 4096, 128),           # 15 x 16 = 240 tiles of 256 x 256: 256 x 128 tiles
    (4096, 4096 - 3, 128),       # 256 tiles of 256 x 256, ragged N: the 256 x 256 kernel
    (1024, 2048, 256),           # 64 tiles of 256 x 128 and 256 of 128 x 64: 128 x 64 tiles
    (1024, 2049, 256),           # 264 of 128 x 64: 256 x 64 tiles
    (1000, 1500, 384),           # 192 of 128 x 64, ragged M and N: 128 x 64 tiles
    (100, 700, 128),             # one tile row shorter than 128: 128 x 64 tiles
])
def test_tensor_gemm_tile_width_boundaries(sq, mnk):
    M, N, K = mnk
    announce("tensor gemm tile-width boundary", mnk)
    rng = np.random.default_rng(M + 5 * N + K)
    A, B = _codes(rng, (M, K), 0), _codes(rng, (N, K), 1)
    sa, sb = np.float32(0.03), np.float32(0.002)
    C = sq.fp8_gemm(_t(A), 0, _scal(sa), 0, _t(B), 1, _scal(sb), 0, sq.OUT_BF16)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.choice(M, min(M, 24), replace=False), [0, M - 1]]))
    Cr, S, G = og.gemm_ref(A, 0, sa, og.TENSOR, B, 1, sb, og.TENSOR, rows=rows)
    check_gemm(np_of(C)[rows], Cr, S, G, K, "tensor", True, f"tile-width boundary {mnk}")


@pytest.mark.parametrize("out", [0, 1])
@pytest.mark.parametrize("mnk", [(256, 256, 256), (200, 300, 512), (1, 130, 128), (129, 257, 384)])
def test_blockwise_gemm(sq, out, mnk):
    M, N, K = mnk
    announce("blockwise gemm", out, mnk)
    rng = np.random.default_rng(M + 13 * N + K)
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp2(rng.integers(-6, 6, (M, 1))).astype(np.float32)
    x.flat[rng.integers(0, x.size, max(1, x.size // 1000))] *= 100.0
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A, sa = oq.quantize_tile_1x128(x, 0)
    B, sb = oq.quantize_block_128x128(w, 0)
    C = sq.fp8_gemm(_t(A), 0, _t(sa), sq.FP8_SCALE_TILE_1x128, _t(B), 0, _t(sb), sq.FP8_SCALE_BLOCK_128x128, out)
    torch.cuda.synchronize()
    Cr, S, G = og.gemm_ref(A, 0, sa, og.TILE_1x128, B, 0, sb, og.BLOCK_128x128)
    check_gemm(np_of(C), Cr, S, G, K, "block", out == 1, f"blockwise {mnk} out{out}")


@pytest.mark.parametrize("out", [0, 1])
@pytest.mark.parametrize("mnk", [(256, 256, 256), (100, 200, 384), (1, 1, 128), (257, 129, 512)])
def test_mx_gemm(sq, out, mnk):
    M, N, K = mnk
    announce("mx gemm", out, mnk)
    rng = np.random.default_rng(M + 17 * N + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-30, 30, (M, K // 32)).repeat(32, 1))).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    A, ea = oq.quantize_mx_1x32(x, 0)
    B, eb = oq.quantize_mx_1x32(w, 0)
    C = sq.fp8_gemm(_t(A), 0, _t(ea.T), sq.FP8_SCALE_MX_1x32, _t(B), 0, _t(eb.T), sq.FP8_SCALE_MX_1x32, out)
    torch.cuda.synchronize()
    Cr, S, G = og.gemm_ref(A, 0, ea, og.MX_1x32, B, 0, eb, og.MX_1x32)
    check_gemm(np_of(C), Cr, S, G, K, "mx", out == 1, f"mx {mnk} out{out}")


# Shapes with at least 256 tiles of 256 x 256, so that per-tensor scaling reaches the
# large-tile kernel too: ragged edges in M and N, and 1, 3, 9 and 2 K stages of 128 (fewer
# than the stages its loads run ahead, odd counts, a count the unrolled loop does not divide).
BIG_CASES = [(4096, 4352, 128), (4100, 4036, 384), (4296, 4036, 1152), (4052, 4100, 256)]


@pytest.mark.parametrize("mnk", BIG_CASES)
@pytest.mark.parametrize("mode", ["tensor", "mx"])
def test_large_tile_kernel(sq, mnk, mode):
    M, N, K = mnk
    announce("large-tile gemm", mode, mnk)
    rng = np.random.default_rng(M + N + K)
    if mode == "tensor":
        A, B = _codes(rng, (M, K), 1, True), _codes(rng, (N, K), 0, True)
        sa, sb = np.float32(0.0123), np.float32(0.0456)
        C = sq.fp8_gemm(_t(A), 1, _scal(sa), 0, _t(B), 0, _scal(sb), 0, sq.OUT_BF16)
        torch.cuda.synchronize()
        r = np.sort(rng.choice(M, 256, replace=False))
        r[-1] = M - 1
        Cr, S, G = og.gemm_ref(A, 1, sa, og.TENSOR, B, 0, sb, og.TENSOR, rows=r)
        check_gemm(np_of(C)[r], Cr, S, G, K, "tensor", True, f"large tensor {mnk}")
    else:
        x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 8, (M, K // 32)).repeat(32, 1))).astype(np.float32)
        w = rng.standard_normal((N, K)).astype(np.float32)
        A, ea = oq.quantize_mx_1x32(x, 0)
        B, eb = oq.quantize_mx_1x32(w, 0)
        C = sq.fp8_gemm(_t(A), 0, _t(ea.T), sq.FP8_SCALE_MX_1x32, _t(B), 0, _t(eb.T), sq.FP8_SCALE_MX_1x32,
                        sq.OUT_F32)
        torch.cuda.synchronize()
        r = np.sort(rng.choice(M, 256, replace=False))
        r[-1] = M - 1
        Cr, S, G = og.gemm_ref(A, 0, ea, og.MX_1x32, B, 0, eb, og.MX_1x32, rows=r)
        check_gemm(np_of(C)[r], Cr, S, G, K, "mx", False, f"large mx {mnk}")


# Blockwise shapes with many 256 x 128 tiles on the large-tile blockwise kernel:
# ragged M and N (N odd takes the unpaired epilogue), K steps fewer than and not a multiple
# of the pipeline depth, and a long K (112 steps).
BIG_BLOCK_CASES = [(2085, 4100, 384), (2048, 4097, 1152), (4096, 2304, 256), (1300, 3000, 128), (300, 520, 14336)]


@pytest.mark.parametrize("out", [0, 1])
@pytest.mark.parametrize("mnk", BIG_BLOCK_CASES)
def test_large_tile_blockwise(sq, mnk, out):
    M, N, K = mnk
    announce("large-tile blockwise gemm", out, mnk)
    rng = np.random.default_rng(M + 3 * N + K)
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp2(rng.integers(-6, 6, (M, 1))).astype(np.float32)
    x.flat[rng.integers(0, x.size, max(1, x.size // 1000))] *= 100.0
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[:, :128] *= 50.0  # one weight block column with a much larger scale
    A, sa = oq.quantize_tile_1x128(x, 0)
    B, sb = oq.quantize_block_128x128(w, 0)
    C = sq.fp8_gemm(_t(A), 0, _t(sa), sq.FP8_SCALE_TILE_1x128, _t(B), 0, _t(sb), sq.FP8_SCALE_BLOCK_128x128, out)
    torch.cuda.synchronize()
    r = np.sort(rng.choice(M, 192, replace=False))
    r[-1] = M - 1
    Cr, S, G = og.gemm_ref(A, 0, sa, og.TILE_1x128, B, 0, sb, og.BLOCK_128x128, rows=r)
    check_gemm(np_of(C)[r], Cr, S, G, K, "block", out == 1, f"large blockwise {mnk} out{out}")


@pytest.mark.parametrize("mode", ["tensor", "mx", "block"])
def test_long_k(sq, mode):
    """K = 65536 (512 promotion blocks, 1024 K steps of the 256x256 kernel) at a small output."""
    M, N, K = 256, 260 if mode != "mx" else 256, 65536
    announce("long K", mode, (M, N, K))
    rng = np.random.default_rng(65536 + len(mode))
    if mode == "tensor":
        A, B = _codes(rng, (M, K), 0, True), _codes(rng, (N, K), 0, True)
        sa, sb = np.float32(0.01), np.float32(0.02)
        C = sq.fp8_gemm(_t(A), 0, _scal(sa), 0, _t(B), 0, _scal(sb), 0, sq.OUT_F32)
        torch.cuda.synchronize()
        Cr, S, G = og.gemm_ref(A, 0, sa, og.TENSOR, B, 0, sb, og.TENSOR)
    elif mode == "mx":
        x = rng.standard_normal((M, K)).astype(np.float32)
        w = rng.standard_normal((N, K)).astype(np.float32)
        A, ea = oq.quantize_mx_1x32(x, 0)
        B, eb = oq.quantize_mx_1x32(w, 0)
        C = sq.fp8_gemm(_t(A), 0, _t(ea.T), sq.FP8_SCALE_MX_1x32, _t(B), 0, _t(eb.T), sq.FP8_SCALE_MX_1x32,
                        sq.OUT_F32)
        torch.cuda.synchronize()
        Cr, S, G = og.gemm_ref(A, 0, ea, og.MX_1x32, B, 0, eb, og.MX_1x32)
    else:
        x = rng.standard_normal((M, K)).astype(np.float32)
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        A, sa = oq.quantize_tile_1x128(x, 0)
        B, sb = oq.quantize_block_128x128(w, 0)
        C = sq.fp8_gemm(_t(A), 0, _t(sa), sq.FP8_SCALE_TILE_1x128, _t(B), 0, _t(sb), sq.FP8_SCALE_BLOCK_128x128,
                        sq.OUT_F32)
        torch.cuda.synchronize()
        Cr, S, G = og.gemm_ref(A, 0, sa, og.TILE_1x128, B, 0, sb, og.BLOCK_128x128)
    check_gemm(np_of(C), Cr, S, G, K, "block" if mode == "block" else mode, False, f"long K {mode}")


@pytest.mark.parametrize("M,N", [(64, 64), (512, 520)])
def test_all_maximum_codes_sum_exactly(sq, M, N):
    """Every code 448 (0x7E) or -448 (0xFE): each product is +-200704 = +-49 * 2^12 and any
    partial sum is a multiple of it below 2^24 * 2^12, so the result is exact: C = 200704 * (K
    with signs)."""
    K = 1024
    announce("all maximum codes", (M, N, K))
    A = np.full((M, K), 0x7E, np.uint8)
    A[1::2, :] = 0xFE  # odd rows negative
    B = np.full((N, K), 0x7E, np.uint8)
    B[:, : K // 4] = 0xFE  # a quarter of each column negative
    C = sq.fp8_gemm(_t(A), 0, _scal(1.0), 0, _t(B), 0, _scal(1.0), 0, sq.OUT_F32)
    torch.cuda.synchronize()
    row_sign = np.where(np.arange(M) % 2 == 1, -1.0, 1.0)[:, None]
    want = row_sign * 200704.0 * (K - 2 * (K // 4)) * np.ones((1, N))
    assert np.array_equal(np_of(C), want.astype(np.float32))


def _ieee_rows(Ad, Bd, rows):
    """The definition's sums for the given rows, elementwise in float64 (IEEE: a NaN product,
    inf x 0 or inf - inf give NaN)."""
    with np.errstate(invalid="ignore", over="ignore"):
        return np.stack([np.sum(Ad[m][None, :] * Bd, axis=1) for m in rows])


@pytest.mark.parametrize("route", [("large", 4096, 4096), ("narrow", 256, 512), ("small", 2, 96)])
def test_nan_inf_codes_propagate(sq, route):
    """E5M2 infinities and NaN codes in A, E4M3 NaN codes and zero columns in B: outputs are
    NaN exactly where the definition's sum is NaN and +-inf where it is +-inf."""
    name, M, N = route
    K = 256
    announce("nan/inf codes", name, (M, N, K))
    rng = np.random.default_rng(404)
    A = _codes(rng, (M, K), 1)  # E5M2
    B = _codes(rng, (N, K), 0)  # E4M3
    PINF, NINF, NAN5, NAN4 = 0x7C, 0xFC, 0x7F, 0x7F
    rows = np.arange(min(M, 48))
    for m in rows:
        kind, k = m % 6, (m * 37) % K
        if kind == 0:
            A[m, k] = NAN5
        elif kind == 1:
            A[m, k] = PINF
        elif kind == 2:
            A[m, k] = NINF
        elif kind == 3:
            A[m, k], A[m, (k + 100) % K] = PINF, NINF
        elif kind == 4:
            A[m, k], A[m, (k + 9) % K] = PINF, PINF
    B[::5, :] = np.where(np.arange(K)[None, :] % 37 == 0, 0, B[::5, :])  # zeros under some infinities
    B[3 % N, 11] = NAN4
    sa, sb = np.float32(0.5), np.float32(0.25)
    C = np_of(sq.fp8_gemm(_t(A), 1, _scal(sa), 0, _t(B), 0, _scal(sb), 0, sq.OUT_F32))[rows].astype(np.float64)
    torch.cuda.synchronize()
    want = _ieee_rows(og.dequant(A, 1, og.TENSOR, sa), og.dequant(B, 0, og.TENSOR, sb), rows)
    assert np.isnan(want).any() and np.isinf(want).any()
    assert np.array_equal(np.isnan(C), np.isnan(want)), f"{name}: NaN positions differ"
    inf = np.isinf(want)
    assert np.array_equal(np.isinf(C), inf) and np.array_equal(np.sign(C[inf]), np.sign(want[inf])), \
        f"{name}: infinities differ"
