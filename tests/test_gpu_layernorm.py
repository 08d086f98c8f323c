"""GPU parity of fp8_layernorm_quantize against oracle/layernorm.py.

The kernel computes the norm in fp32 (row sums over the lanes' registers, then across the
wave), the oracle in float64, so y differs by rounding; the codes (and the current scales
derived from y) are decided by the kernel's fp32 y.  ln_bound() derives a per-element bound
on |y_gpu - y| from the number of fp32 roundings each quantity sees; the test then places
every scale and code in the interval the bound allows: amax in [max(|y| - e), max(|y| + e)],
the scale (monotone in amax) between the scales of the interval's ends, and each code between
the codes of the smallest and largest products the intervals allow.  Rows whose y is exact on
both sides (constant rows: y = beta) are compared bit for bit."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import DEV, announce, np_of  # noqa: E402
from oracle import fp8 as ofp8, layernorm as oln, quantize as oq, recipe as orc  # noqa: E402

U = 2.0 ** -24
EPS = float(np.float32(1e-5))  # the fp32 eps the kernel receives


@pytest.fixture(scope="module")
def sq():
    import scaled_quantize_gemm_amd as m

    return m


def ln_bound(x, gamma, beta, eps):
    """(y, mean, rs, e_y, e_mean, rel_rs): oracle values and bounds on the kernel's errors.

    Every fp32 sum a row goes through (a lane's sequential adds, at most cols/64 + 8, then 6
    shuffle levels and a divide) rounds at most c = (cols/64 + 16) u relative to the sum of
    magnitudes, u = 2^-24.  Then: mean off by e_mean = c (mean|x| + |mean|); each deviation
    d by delta = e_mean + u|d|; the sum of squares by sum(2|d| delta + delta^2) + c sum((|d| +
    delta)^2); var + eps by that / cols + 2u (var + eps); rs relatively by 0.6 e_v / (var + eps)
    + 3u (square root and divide correctly rounded); y = fma(d rs, gamma, beta) by
    |gamma| rs (delta (1 + rel) + |d| rel + u |d| (1 + rel)) plus u |y|.  Doubled for margin."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[1]
    y, mean, rs = oln.layernorm_ref(x, gamma, beta, eps)
    c = (n / 64 + 16) * U
    d = x - mean[:, None]
    e_mean = c * (np.abs(x).mean(axis=1) + np.abs(mean))
    delta = e_mean[:, None] + U * np.abs(d)
    e_ssq = (2 * np.abs(d) * delta + delta ** 2).sum(axis=1) + c * ((np.abs(d) + delta) ** 2).sum(axis=1)
    v = (d * d).sum(axis=1) / n + eps
    e_v = e_ssq / n + 2 * U * v
    rel = 0.6 * e_v / v + 3 * U
    g = np.abs(np.asarray(gamma, dtype=np.float64))[None, :]
    r = rs[:, None]
    e_prod = g * r * (delta * (1 + rel[:, None]) + np.abs(d) * rel[:, None] + U * np.abs(d) * (1 + rel[:, None]))
    e_y = 2 * (e_prod + U * (np.abs(y) + e_prod))
    return y, mean, rs, e_y, 2 * e_mean, 2 * rel


def _f32_interval(lo, hi):
    """fp32 values a kernel's fp32 quantity in [lo, hi] can round to: [rn(lo), rn(hi)]."""
    return np.asarray(lo, dtype=np.float64).astype(np.float32), np.asarray(hi, dtype=np.float64).astype(np.float32)


def _products(ylo, yhi, slo, shi):
    c = np.stack([ylo * slo, ylo * shi, yhi * slo, yhi * shi])
    return c.min(axis=0), c.max(axis=0)


def _codes_between(codes, plo, phi, fmt, label):
    with np.errstate(over="ignore"):
        lo = ofp8.decode(ofp8.encode(plo.astype(np.float32), fmt), fmt)
        hi = ofp8.decode(ofp8.encode(phi.astype(np.float32), fmt), fmt)
    d = ofp8.decode(codes, fmt)
    ok = (lo <= d) & (d <= hi)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{label}: {int((~ok).sum())} codes outside; first {i}: {d[i]} not in [{lo[i]}, {hi[i]}]")


def check_ln(sq, x, gamma, beta, fmt, gran, label, rows=None, scale=None, amax0=0.0):
    """Run the kernel on device copies of x / gamma / beta (torch tensors) and check rows."""
    announce("layernorm", label)
    R, C = x.shape
    xd, gd = x.to(DEV), gamma.to(DEV)
    bd = None if beta is None else beta.to(DEV)
    mu, rsg = torch.empty(R, device=DEV), torch.empty(R, device=DEV)
    slot = torch.tensor([amax0], dtype=torch.float32, device=DEV)
    sc = None if scale is None else torch.tensor([scale], dtype=torch.float32, device=DEV)
    q, sinv = sq.fp8_layernorm_quantize(xd, gd, bd, EPS, fmt, gran, scale=sc, amax_slot=slot, mu=mu, rsigma=rsg)
    torch.cuda.synchronize()
    r = np.arange(R) if rows is None else rows
    xo = x.float().numpy()[r]
    go = gamma.float().numpy()
    bo = None if beta is None else beta.float().numpy()
    y, mean, rs, e, e_mean, rel = ln_bound(xo, go, bo, EPS)
    np_mu, np_rs = np_of(mu)[r], np_of(rsg)[r]
    assert np.all(np.abs(np_mu - mean) <= e_mean), (label, "mean")
    assert np.all(np.abs(np_rs - rs) <= rel * rs), (label, "rsigma")
    codes = np_of(q)[r]
    fmax = ofp8.FMAX[fmt]
    ylo, yhi = y - e, y + e
    if gran == oln.TENSOR:
        s = np.float64(np.float32(scale))
        _codes_between(codes, ylo * s, yhi * s, fmt, label)
        a = float(np_of(slot)[0])
        lo_a = max(amax0, float((np.abs(y) - e).max()))
        assert a >= lo_a, (label, a, lo_a)
        if rows is None:
            assert a <= max(amax0, float((np.abs(y) + e).max())) * (1 + U), (label, a)
        return
    run = 128 if gran == oln.TILE_1x128 else 32
    alo = np.maximum(np.abs(y) - e, 0).reshape(len(r), C // run, run).max(axis=2)
    ahi = (np.abs(y) + e).reshape(len(r), C // run, run).max(axis=2)
    alo32, ahi32 = _f32_interval(alo, ahi)
    assert np.all(alo32 > 0), "runs with a zero amax are checked bit-exactly elsewhere"
    if gran == oln.TILE_1x128:
        s_hi, sinv_lo = orc.current_scale(alo32, fmt)
        s_lo, sinv_hi = orc.current_scale(ahi32, fmt)
        got = np_of(sinv).T[r]  # [rows][runs]
        ok = (sinv_lo <= got) & (got <= sinv_hi)
        assert ok.all(), (label, "scale_inv", np.argwhere(~ok)[:3])
    else:
        e_lo, e_hi = orc.mx_exponent(alo32, fmt), orc.mx_exponent(ahi32, fmt)
        got = np_of(sinv).T[r]
        ok = (e_lo <= got) & (got <= e_hi)
        assert ok.all(), (label, "e8m0", np.argwhere(~ok)[:3])
        s_lo = np.exp2(-(e_hi.astype(np.float64) - 127))
        s_hi = np.exp2(-(e_lo.astype(np.float64) - 127))
    slo = np.repeat(np.asarray(s_lo, np.float64), run, axis=1)
    shi = np.repeat(np.asarray(s_hi, np.float64), run, axis=1)
    plo, phi = _products(ylo, yhi, slo, shi)
    _codes_between(codes, plo, phi, fmt, label)
    # the codes never exceed the format: the run's largest code is at most fmax
    assert np.all(np.abs(ofp8.decode(codes, fmt)) <= fmax)


def _inputs(rng, R, C, dtype, offset=0.0):
    x = torch.from_numpy((rng.standard_normal((R, C)) + offset).astype(np.float32)).to(dtype)
    g = torch.from_numpy((1 + 0.1 * rng.standard_normal(C)).astype(np.float32)).to(dtype)
    b = torch.from_numpy((0.1 * rng.standard_normal(C)).astype(np.float32)).to(dtype)
    return x, g, b


SHAPES = [(2048, 768), (37, 8192), (5, 128), (300, 2176), (64, 4096)]


@pytest.mark.parametrize("gran", [oln.TENSOR, oln.TILE_1x128, oln.MX_1x32])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fmt,dtype", [(0, torch.bfloat16), (1, torch.float32), (0, torch.float32)])
def test_layernorm_quantize(sq, gran, shape, fmt, dtype):
    rng = np.random.default_rng(shape[0] * 3 + shape[1] + gran + 5 * fmt)
    x, g, b = _inputs(rng, *shape, dtype)
    scale = ofp8.FMAX[fmt] / 4.0  # |y| > 4 saturates
    check_ln(sq, x, g, b, fmt, gran, f"{shape} gran{gran} fmt{fmt} {dtype}", scale=scale)


@pytest.mark.parametrize("gran", [oln.TENSOR, oln.TILE_1x128, oln.MX_1x32])
def test_layernorm_offset_rows_and_no_beta(sq, gran):
    """Rows with mean 100 (cancellation in x - mean) and no beta."""
    rng = np.random.default_rng(9)
    x, g, _ = _inputs(rng, 96, 1024, torch.float32, offset=100.0)
    check_ln(sq, x, g, None, 0, gran, f"offset gran{gran}", scale=448.0 / 4.0)


def test_layernorm_tensor_ragged_cols(sq):
    """cols a multiple of 8 only (per-tensor scaling): 200 columns, partial chunk groups."""
    rng = np.random.default_rng(10)
    x, g, b = _inputs(rng, 3, 200, torch.bfloat16)
    check_ln(sq, x, g, b, 0, oln.TENSOR, "cols 200", scale=448.0 / 4.0, amax0=0.5)


@pytest.mark.parametrize("gran", [oln.TENSOR, oln.TILE_1x128, oln.MX_1x32])
def test_layernorm_constant_rows_are_exact(sq, gran):
    """Constant rows: x - mean is exactly 0 on both sides, so y = beta exactly and the codes
    and scales equal the oracle's bit for bit (zero beta: the zero-amax rules)."""
    announce("layernorm constant rows", gran)
    C = 256
    x = torch.full((4, C), 3.0, dtype=torch.float32)
    x[1] = -7.0
    g = torch.full((C,), 2.0)
    b = torch.from_numpy(np.linspace(-3, 3, C).astype(np.float32))
    b[:128] = 0.0  # a zero run
    q, sinv = sq.fp8_layernorm_quantize(x.to(DEV), g.to(DEV), b.to(DEV), EPS, 0, gran,
                                        scale=torch.tensor([100.0], device=DEV))
    torch.cuda.synchronize()
    want = oln.layernorm_quantize(x.numpy(), g.numpy(), b.numpy(), EPS, 0, gran, scale=100.0)
    assert np.array_equal(np_of(q), want[0])
    if gran == oln.TILE_1x128:  # both [cols/128][rows]
        assert np.array_equal(np_of(sinv), want[1])
    elif gran == oln.MX_1x32:  # kernel [cols/32][rows], oracle [rows][cols/32]
        assert np.array_equal(np_of(sinv).T, want[1])


def test_layernorm_empty_and_errors(sq):
    x = torch.empty((0, 768), device=DEV)
    g = torch.ones(768, device=DEV)
    q, _ = sq.fp8_layernorm_quantize(x, g, None, EPS, 0, sq.FP8_SCALE_TENSOR, scale=torch.ones(1, device=DEV))
    assert q.shape == (0, 768)
    x = torch.zeros((4, 768), device=DEV)
    with pytest.raises(sq.Fp8Error) as e:
        sq.fp8_layernorm_quantize(x, g, None, EPS, 0, sq.FP8_SCALE_BLOCK_128x128)
    assert e.value.code == sq.FP8_ERR_ARG
    x = torch.zeros((4, 8200), device=DEV)
    with pytest.raises(sq.Fp8Error) as e:
        sq.fp8_layernorm_quantize(x, torch.ones(8200, device=DEV), None, EPS, 0, sq.FP8_SCALE_TENSOR,
                                  scale=torch.ones(1, device=DEV))
    assert e.value.code == sq.FP8_ERR_SHAPE


def test_workload4_input_layernorm(sq):
    """The FC1 input X [8192x4096] bf16 through a LayerNorm: per-tensor (delayed scale, amax
    recorded) and 1x128 tiles; sampled rows against the oracle."""
    import workloads

    X, _, _ = workloads.w4_inputs()
    rng = np.random.default_rng(12)
    g = torch.from_numpy((1 + 0.1 * rng.standard_normal(4096)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy((0.1 * rng.standard_normal(4096)).astype(np.float32)).to(torch.bfloat16)
    r = np.sort(rng.choice(8192, 64, replace=False))
    for gran in (oln.TENSOR, oln.TILE_1x128):
        check_ln(sq, X, g, b, 0, gran, f"workload4 LN gran{gran}", rows=r, scale=448.0 / 5.0)


def test_layernorm_mx_rows_not_multiple_of_group(sq):
    """MX at 1000 rows (not a multiple of the 8-row groups) and bf16 gamma without beta."""
    rng = np.random.default_rng(13)
    x, g, _ = _inputs(rng, 1000, 1536, torch.bfloat16)
    check_ln(sq, x, g, None, 1, oln.MX_1x32, "mx 1000x1536 no beta")


def _ln_random_cases(n=24, seed=77):
    """Seeded random LayerNorm shapes: rows 1..3000, cols a multiple of the granularity's run up
    to 8192, both formats, both input types, with and without beta, offset rows."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        gran = [oln.TENSOR, oln.TILE_1x128, oln.MX_1x32][i % 3]
        run = {oln.TENSOR: 8, oln.TILE_1x128: 128, oln.MX_1x32: 32}[gran]
        cols = run * int(rng.integers(1, 8192 // run + 1))
        rows = int(rng.integers(1, 3001))
        out.append((gran, rows, cols, int(rng.integers(0, 2)), bool(rng.random() < 0.5), bool(rng.random() < 0.7),
                    float(rng.choice([0.0, 3.0, 50.0])), 500 + i))
    return out


@pytest.mark.parametrize("case", _ln_random_cases(), ids=lambda c: f"g{c[0]}-{c[1]}x{c[2]}-f{c[3]}")
def test_layernorm_random_shapes(sq, case):
    gran, rows, cols, fmt, bf16, with_beta, offset, seed = case
    rng = np.random.default_rng(seed)
    x, g, b = _inputs(rng, rows, cols, torch.bfloat16 if bf16 else torch.float32, offset=offset)
    check_ln(sq, x, g, b if with_beta else None, fmt, gran, f"random {case}", scale=ofp8.FMAX[fmt] / 4.0)
