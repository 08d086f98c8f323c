"""GPU parity of fp8_cast_transpose: q, qT and amax bit-exact against the oracle."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import DEV, announce, assert_codes_equal, assert_f32_bits_equal, f32_np, np_of  # noqa: E402
from oracle import fp8 as ofp8, quantize as oq  # noqa: E402


@pytest.fixture(scope="module")
def sq():
    import scaled_quantize_gemm_amd as m

    return m


# 128-aligned shapes take the 128 x 128 kernel, the others the 64 x 64 kernel; (1408, 384) and
# (1152, 640) have 11 and 9 tile rows, so the 128 x 128 kernel's last band of 8 tile rows is partial.
# Both launches cap their grids at the blocks resident at once (3 per CU for the 128 x 128
# kernel's per-tensor mode, 8 for the 64 x 64 one), the blocks looping over tiles: (4096, 3200)
# has 800 tiles of 128 x 128 and (3000, 2900) 2162 of 64 x 64, so some blocks take two tiles
SHAPES = [(1, 1), (64, 64), (128, 192), (100, 37), (3, 1000), (200, 136), (257, 130), (2048, 768), (64, 2304),
          (128, 128), (256, 384), (384, 128), (1408, 384), (1152, 640), (4096, 3200), (3000, 2900)]


@pytest.mark.parametrize("fmt", [ofp8.E4M3, ofp8.E5M2])
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_cast_transpose_matches_oracle(sq, fmt, bf16, shape):
    announce("cast_transpose", ofp8.fmt_name(fmt), "bf16" if bf16 else "f32", shape)
    rows, cols = shape
    rng = np.random.default_rng(rows * 1009 + cols)
    x = (rng.standard_normal(shape) * 3.0).astype(np.float32)
    if rows * cols > 10:
        x.flat[rng.integers(0, x.size, 3)] = [np.inf, -0.0, 1e30]
    xt = torch.from_numpy(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
    scale = np.float32(448.0 / 9.0) if fmt == ofp8.E4M3 else np.float32(57344.0 / 9.0)
    s = torch.tensor([scale], device=DEV)
    slot = torch.zeros(1, device=DEV)
    q, qT = sq.fp8_cast_transpose(xt.to(DEV), fmt, s, amax_slot=slot)
    torch.cuda.synchronize()
    oq_, oqT, oa = oq.cast_transpose(f32_np(xt), scale, fmt)
    assert_codes_equal(np_of(q), oq_, "q")
    assert_codes_equal(np_of(qT), oqT, "qT")
    assert_f32_bits_equal(np_of(slot), [oa], "amax")


@pytest.mark.parametrize("shape", [(64, 64), (256, 256)])
def test_cast_transpose_nan_propagates(sq, shape):
    announce("cast_transpose NaN", shape)
    x = np.ones(shape, np.float32)
    x[10, 20] = np.nan
    x[11, 21] = -np.nan
    s = torch.ones(1, device=DEV)
    slot = torch.zeros(1, device=DEV)
    q, qT = sq.fp8_cast_transpose(torch.from_numpy(x).to(DEV), sq.FP8_E4M3, s, amax_slot=slot)
    torch.cuda.synchronize()
    oq_, oqT, oa = oq.cast_transpose(x, np.float32(1.0), ofp8.E4M3)
    assert_codes_equal(np_of(q), oq_, "q")
    assert_codes_equal(np_of(qT), oqT, "qT")
    assert np.isnan(np_of(slot)[0])


def test_cast_transpose_full_size_sampled(sq):
    """Workload 4's gradient dY [8192 x 14336] in E5M2, launch as the bench runs it; sampled rows / columns."""
    import workloads

    announce("cast_transpose full size dY 8192x14336 E5M2")
    _, _, dy = workloads.w4_inputs()
    s = torch.tensor([np.float32(57344.0) / np.float32(5e-4)], device=DEV)
    slot = torch.zeros(1, device=DEV)
    q, qT = sq.fp8_cast_transpose(dy.to(DEV), sq.FP8_E5M2, s, amax_slot=slot)
    torch.cuda.synchronize()
    x = f32_np(dy)
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(x.shape[0], 48, replace=False))
    cols = np.sort(rng.choice(x.shape[1], 48, replace=False))
    sc = np.float32(s.item())
    assert_codes_equal(np_of(q[torch.from_numpy(rows).to(DEV)]), oq.quantize_tensor(x[rows], sc, ofp8.E5M2)[0],
                       "q rows")
    assert_codes_equal(np_of(qT[torch.from_numpy(cols).to(DEV)]),
                       oq.quantize_tensor(np.ascontiguousarray(x[:, cols].T), sc, ofp8.E5M2)[0], "qT rows")
    assert_f32_bits_equal(np_of(slot), [np.abs(x).max()], "amax")
