"""GPU parity of the quantizers against the oracle: codes, amax and scales bit-exact."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import DEV, announce, assert_codes_equal, assert_f32_bits_equal, f32_np, np_of  # noqa: E402
from oracle import fp8 as ofp8, quantize as oq, recipe as orc  # noqa: E402

FMTS = [ofp8.E4M3, ofp8.E5M2]


@pytest.fixture(scope="module")
def sq():
    import scaled_quantize_gemm_amd as m

    ok, why = m.fp8_device_check(0)
    assert ok, why
    return m


def _special_f32(n, seed):
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    sp = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001,
                   0x00000001, 0x80000001, 0x43E00000, 0xC3E00000, 0x43E80000, 0x47600000, 0x47700000],
                  dtype=np.uint32)
    k = min(n, len(sp))
    u[:k] = sp[:k]
    return u.view(np.float32)


def _tensor_quant(sq, x_t, scale, fmt):
    s = torch.tensor([scale], dtype=torch.float32, device=DEV)
    slot = torch.zeros(1, dtype=torch.float32, device=DEV)
    q, _ = sq.fp8_quantize(x_t, fmt, sq.FP8_SCALE_TENSOR, scale=s, amax_slot=slot)
    torch.cuda.synchronize()
    return np_of(q), np_of(slot)[0]


@pytest.mark.parametrize("fmt", FMTS)
def test_tensor_cast_every_bf16_pattern(sq, fmt):
    """All 65536 bf16 inputs x several scales, incl. NaN / inf / subnormal / -0 / overflow."""
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    xb = torch.from_numpy(bits.copy()).to(torch.bfloat16).view(256, 256)
    for scale in [1.0, float(np.float32(448.0) / np.float32(240.0)), 2.0 ** -10, 3.0e4, 3.4e38]:
        announce("tensor cast bf16 patterns", ofp8.fmt_name(fmt), scale)
        q, amax = _tensor_quant(sq, xb.to(DEV), scale, fmt)
        oq_, oa = oq.quantize_tensor(f32_np(xb), np.float32(scale), fmt)
        assert_codes_equal(q, oq_, f"bf16 patterns scale={scale}")
        assert np.isnan(amax) and np.isnan(oa)
    finite = bits[np.isfinite(bits)]
    xf = torch.from_numpy(finite.copy()).to(torch.bfloat16)
    q, amax = _tensor_quant(sq, xf.to(DEV), 1.0, fmt)
    oq_, oa = oq.quantize_tensor(f32_np(xf), np.float32(1.0), fmt)
    assert_codes_equal(q, oq_, "finite bf16")
    assert_f32_bits_equal([amax], [oa], "amax")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n", [1, 15, 16, 17, 4096 + 7, 1_000_003])
def test_tensor_cast_random_f32_bits_ragged(sq, fmt, n):
    announce("tensor cast random f32", ofp8.fmt_name(fmt), n)
    x = _special_f32(n, 100 + n)
    for scale in [1.0, 0.37, 1.0e3]:
        q, amax = _tensor_quant(sq, torch.from_numpy(x.copy()).to(DEV), scale, fmt)
        oq_, oa = oq.quantize_tensor(x, np.float32(scale), fmt)
        assert_codes_equal(q, oq_, f"n={n} scale={scale}")
        assert_f32_bits_equal([amax], [oa], "amax")
    # finite data: amax bit-exact; amax slot accumulates with max across calls
    xf = np.where(np.isfinite(x), x, 1.0).astype(np.float32)
    s = torch.tensor([2.0], dtype=torch.float32, device=DEV)
    slot = torch.full((1,), 1e-3, dtype=torch.float32, device=DEV)
    sq.fp8_quantize(torch.from_numpy(xf).to(DEV), fmt, sq.FP8_SCALE_TENSOR, scale=s, amax_slot=slot)
    sq.fp8_quantize(torch.from_numpy(xf * 0.5).to(DEV), fmt, sq.FP8_SCALE_TENSOR, scale=s, amax_slot=slot)
    torch.cuda.synchronize()
    assert_f32_bits_equal(np_of(slot), [max(np.float32(1e-3), orc.amax(xf))], "running amax")


def _blocky_data(rows, cols, seed, specials=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, (rows, 1))).astype(np.float32)
    if rows > 2 and cols >= 256:
        x[1, :] = 0.0  # a zero row: unit scales
        x[2, 5] *= 1000.0  # an outlier
    if specials and rows > 4 and cols >= 256:
        x[3, 7] = np.nan
        x[4, 130] = np.inf
        x[0, 3] = -0.0
        x[0, 200] = 1e-41
    return x


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("shape", [(1, 128), (37, 384), (256, 1024), (300, 7168)])
def test_tile_1x128(sq, fmt, bf16, shape):
    announce("tile 1x128", ofp8.fmt_name(fmt), "bf16" if bf16 else "f32", shape)
    x = _blocky_data(*shape, seed=shape[0] + 7 * shape[1])
    xt = torch.from_numpy(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
    q, sinv = sq.fp8_quantize(xt.to(DEV), fmt, sq.FP8_SCALE_TILE_1x128)
    torch.cuda.synchronize()
    oq_, osinv = oq.quantize_tile_1x128(f32_np(xt), fmt)
    assert_codes_equal(np_of(q), oq_, "tile codes")
    assert_f32_bits_equal(np_of(sinv), osinv, "tile scale_inv")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("shape", [(1, 128), (128, 128), (200, 256), (513, 384)])
def test_block_128x128(sq, fmt, bf16, shape):
    announce("block 128x128", ofp8.fmt_name(fmt), "bf16" if bf16 else "f32", shape)
    x = _blocky_data(*shape, seed=3 * shape[0] + shape[1])
    xt = torch.from_numpy(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
    q, sinv = sq.fp8_quantize(xt.to(DEV), fmt, sq.FP8_SCALE_BLOCK_128x128)
    torch.cuda.synchronize()
    oq_, osinv = oq.quantize_block_128x128(f32_np(xt), fmt)
    assert_codes_equal(np_of(q), oq_, "block codes")
    assert_f32_bits_equal(np_of(sinv), osinv, "block scale_inv")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("shape", [(1, 32), (5, 96), (64, 1024), (333, 160)])
def test_mx_1x32(sq, fmt, bf16, shape):
    announce("mx 1x32", ofp8.fmt_name(fmt), "bf16" if bf16 else "f32", shape)
    rng = np.random.default_rng(shape[0] * 31 + shape[1])
    x = (rng.standard_normal(shape) * np.exp2(rng.integers(-60, 60, (shape[0], shape[1] // 32)).repeat(32, 1)))
    x = x.astype(np.float32)
    if shape[0] > 3 and shape[1] >= 96:
        x[0, :32] = 0.0
        x[1, 40] = np.nan
        x[2, 70] = -np.inf
        x[3, 0] = 1e-40
    xt = torch.from_numpy(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
    q, e8 = sq.fp8_quantize(xt.to(DEV), fmt, sq.FP8_SCALE_MX_1x32)
    torch.cuda.synchronize()
    oq_, oe8 = oq.quantize_mx_1x32(f32_np(xt), fmt)
    assert_codes_equal(np_of(e8).T, oe8, "e8m0 codes (layout [cols/32][rows])")
    assert_codes_equal(np_of(q), oq_, "mx codes")


def test_empty_inputs(sq):
    announce("empty inputs")
    s = torch.ones(1, device=DEV)
    q, _ = sq.fp8_quantize(torch.empty((0, 128), device=DEV), sq.FP8_E4M3, sq.FP8_SCALE_TENSOR, scale=s)
    assert q.shape == (0, 128)
    q, si = sq.fp8_quantize(torch.empty((0, 128), device=DEV), sq.FP8_E4M3, sq.FP8_SCALE_TILE_1x128)
    torch.cuda.synchronize()
    assert q.numel() == 0


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("n", [1, 1000, 65536 * 3 + 5])
def test_quantize_diag_counts(sq, fmt, bf16, n):
    """Saturated / underflowed / NaN counts match the oracle exactly and accumulate across
    calls; codes and amax match fp8_quantize."""
    announce("quantize_diag", ofp8.fmt_name(fmt), "bf16" if bf16 else "f32", n)
    rng = np.random.default_rng(n + 3 * fmt)
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 12, n))).astype(np.float32)
    k = min(n, 6)
    x[:k] = [np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-30][:k]
    xt = torch.from_numpy(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
    xs = f32_np(xt)
    scale = float(np.float32(ofp8.FMAX[fmt]) / np.float32(300.0))  # clips the large tail
    s = torch.tensor([scale], dtype=torch.float32, device=DEV)
    slot = torch.zeros(1, dtype=torch.float32, device=DEV)
    counts = torch.zeros(3, dtype=torch.int64, device=DEV)
    q = sq.fp8_quantize_diag(xt.to(DEV), fmt, s, counts, amax_slot=slot)
    q2 = sq.fp8_quantize_diag(xt.to(DEV), fmt, s, counts)
    torch.cuda.synchronize()
    want = oq.cast_diagnostics(xs, np.float32(scale), fmt)
    assert np_of(counts).tolist() == [2 * w for w in want]
    oq_, oa = oq.quantize_tensor(xs, np.float32(scale), fmt)
    assert_codes_equal(np_of(q).reshape(-1), oq_, "diag codes")
    assert_codes_equal(np_of(q2).reshape(-1), oq_, "diag codes (second call)")
    assert np.isnan(np_of(slot)[0]) == np.isnan(oa)


def _quant_random_cases(n=32, seed=31337):
    """Seeded random shapes for every quantizer and cast-transpose: rows 1..2600, cols a
    multiple of what the granularity needs, both formats and input types."""
    rng = np.random.default_rng(seed)
    kinds = ["tensor", "tile", "block", "mx", "ct", "ct_bw_tile", "ct_bw_block", "tensor"]
    out = []
    for i in range(n):
        kind = kinds[i % len(kinds)]
        need = {"tensor": 1, "ct": 1, "tile": 128, "block": 128, "mx": 32, "ct_bw_tile": 128, "ct_bw_block": 128}[kind]
        rows = int(rng.integers(1, 2601))
        if kind.startswith("ct_bw"):
            rows = 128 * int(rng.integers(1, 21))
        cols = need * int(rng.integers(1, 4097 // need + 1)) if need > 1 else int(rng.integers(1, 4097))
        out.append((kind, rows, cols, int(rng.integers(0, 2)), bool(rng.random() < 0.5), 7000 + i))
    return out


@pytest.mark.parametrize("case", _quant_random_cases(), ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-f{c[3]}")
def test_quantizers_random_shapes(sq, case):
    """Bit-exact codes, scales and amax against the oracle at random shapes."""
    kind, rows, cols, fmt, bf16, seed = case
    announce("random quantizer", case)
    x = _blocky_data(rows, cols, seed=seed)
    xt = torch.from_numpy(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
    xd, xo = xt.to(DEV), f32_np(xt)
    with np.errstate(over="ignore"):
        scale = np.float32(ofp8.FMAX[fmt] / 8.0)
    if kind == "tensor":
        slot = torch.zeros(1, device=DEV)
        q, _ = sq.fp8_quantize(xd, fmt, sq.FP8_SCALE_TENSOR, scale=torch.tensor([scale], device=DEV), amax_slot=slot)
        torch.cuda.synchronize()
        oq_, oa = oq.quantize_tensor(xo, scale, fmt)
        assert_codes_equal(np_of(q).reshape(oq_.shape), oq_, "tensor codes")
        assert_f32_bits_equal(np_of(slot), np.array([oa], np.float32), "tensor amax")
    elif kind == "tile":
        q, s = sq.fp8_quantize(xd, fmt, sq.FP8_SCALE_TILE_1x128)
        torch.cuda.synchronize()
        oq_, os_ = oq.quantize_tile_1x128(xo, fmt)
        assert_codes_equal(np_of(q), oq_, "tile codes")
        assert_f32_bits_equal(np_of(s), os_, "tile scales")
    elif kind == "block":
        q, s = sq.fp8_quantize(xd, fmt, sq.FP8_SCALE_BLOCK_128x128)
        torch.cuda.synchronize()
        oq_, os_ = oq.quantize_block_128x128(xo, fmt)
        assert_codes_equal(np_of(q), oq_, "block codes")
        assert_f32_bits_equal(np_of(s), os_, "block scales")
    elif kind == "mx":
        q, e8 = sq.fp8_quantize(xd, fmt, sq.FP8_SCALE_MX_1x32)
        torch.cuda.synchronize()
        oq_, oe = oq.quantize_mx_1x32(xo, fmt)
        assert_codes_equal(np_of(e8).T, oe, "mx e8m0")
        assert_codes_equal(np_of(q), oq_, "mx codes")
    elif kind == "ct":
        slot = torch.zeros(1, device=DEV)
        q, qT = sq.fp8_cast_transpose(xd, fmt, torch.tensor([scale], device=DEV), amax_slot=slot)
        torch.cuda.synchronize()
        oq_, oqT, oa = oq.cast_transpose(xo, scale, fmt)
        assert_codes_equal(np_of(q), oq_, "ct codes")
        assert_codes_equal(np_of(qT), oqT, "ct transposed codes")
        assert_f32_bits_equal(np_of(slot), np.array([oa], np.float32), "ct amax")
    else:
        gran = sq.FP8_SCALE_TILE_1x128 if kind == "ct_bw_tile" else sq.FP8_SCALE_BLOCK_128x128
        q, s, qT, sT = sq.fp8_cast_transpose_blockwise(xd, fmt, gran)
        torch.cuda.synchronize()
        want = oq.cast_transpose_blockwise(xo, fmt, 1 if gran == sq.FP8_SCALE_TILE_1x128 else 2)
        assert_codes_equal(np_of(q), want[0], "bw codes")
        assert_f32_bits_equal(np_of(s), want[1], "bw scales")
        assert_codes_equal(np_of(qT), want[2], "bw transposed codes")
        assert_f32_bits_equal(np_of(sT), want[3], "bw transposed scales")
