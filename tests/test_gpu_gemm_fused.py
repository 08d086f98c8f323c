"""GPU parity of fp8_gemm_fused (bias, pre-activation copy, GELU / SwiGLU, fp32 / bf16 / FP8
output with amax) against the oracle GEMM followed by oracle/epilogue.py.

Bounds: the pre-activation carries the GEMM bound of gpu_util.gemm_bound plus one fp32
rounding of the bias add; GELU (|gelu'| <= 1.07) and SwiGLU (|silu'| <= 1.1) propagate it,
and their fp32 evaluation adds at most 2^-20 of |v| (GELU) or |g| |u| (SwiGLU).  A bf16
output adds one bf16 ulp.  An FP8 output code is decided by the kernel's fp32 value, which
the bound places in an interval: the code must lie between the oracle codes of the
interval's ends, and the amax between the ends' largest magnitudes."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import DEV, announce, gemm_bound, np_of  # noqa: E402
from oracle import epilogue as oe, fp8 as ofp8, gemm as og, quantize as oq  # noqa: E402

NONE, GELU, SWIGLU = oe.ACT_NONE, oe.ACT_GELU, oe.ACT_SWIGLU
F32, BF16, E4, E5 = 0, 1, 2, 3


@pytest.fixture(scope="module")
def sq():
    import scaled_quantize_gemm_amd as m

    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _scal(v):
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def _operands(sq, rng, mode, M, N, K):
    """Quantised X [M][K] ~ N(0,1) and W [N][K] ~ N(0, 1/K) (pre-activations of order 1) in
    the mode's granularities: (device args, oracle args, bound mode)."""
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    if mode == "tensor":
        sx, sw = np.float32(448.0 / np.abs(x).max()), np.float32(448.0 / np.abs(w).max())
        A, B = oq.quantize_tensor(x, sx, 0)[0], oq.quantize_tensor(w, sw, 0)[0]
        sa, sb = np.float32(1) / sx, np.float32(1) / sw
        dev = (_t(A), _scal(sa), sq.FP8_SCALE_TENSOR, _t(B), _scal(sb), sq.FP8_SCALE_TENSOR)
        orc = (A, sa, og.TENSOR, B, sb, og.TENSOR)
        return dev, orc, "tensor"
    if mode == "mx":
        A, ea = oq.quantize_mx_1x32(x, 0)
        B, eb = oq.quantize_mx_1x32(w, 0)
        dev = (_t(A), _t(ea.T), sq.FP8_SCALE_MX_1x32, _t(B), _t(eb.T), sq.FP8_SCALE_MX_1x32)
        return dev, (A, ea, og.MX_1x32, B, eb, og.MX_1x32), "mx"
    A, sa = oq.quantize_tile_1x128(x, 0)
    if mode == "block":
        B, sb = oq.quantize_block_128x128(w, 0)
        dev = (_t(A), _t(sa), sq.FP8_SCALE_TILE_1x128, _t(B), _t(sb), sq.FP8_SCALE_BLOCK_128x128)
        return dev, (A, sa, og.TILE_1x128, B, sb, og.BLOCK_128x128), "block"
    B, sb = oq.quantize_tile_1x128(w, 0)
    dev = (_t(A), _t(sa), sq.FP8_SCALE_TILE_1x128, _t(B), _t(sb), sq.FP8_SCALE_TILE_1x128)
    return dev, (A, sa, og.TILE_1x128, B, sb, og.TILE_1x128), "block"


def act_bound(pre, e_pre, act):
    """Bound on |y_gpu - y| from the pre-activation bound e_pre."""
    if act == NONE:
        return e_pre
    if act == GELU:
        return 1.07 * e_pre + 2.0 ** -20 * (np.abs(pre) + e_pre)
    g, u = pre[:, 0::2], pre[:, 1::2]
    eg, eu = e_pre[:, 0::2], e_pre[:, 1::2]
    ag, au = np.abs(g) + eg, np.abs(u) + eu
    return 1.1 * eg * au + (np.abs(oe.silu(g)) + 1.1 * eg) * eu + 2.0 ** -20 * ag * au


def check_values(got, want, bound, bf16, label):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    if bf16:
        bound = bound + ofp8.bf16_ulp(np.maximum(np.abs(want), np.abs(got)))
    bad = ~(err <= bound)
    print(f"[fused] {label} max err/bound {float((err / np.where(bound > 0, bound, 1)).max()):.3g}", flush=True)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{label}: {int(bad.sum())} beyond bound; first {i}: gpu={got[i]} ref={want[i]} "
                             f"bound={bound[i]}")


def check_fp8(codes, y, e_y, scale, fmt, label):
    lo = ofp8.decode(oe.fp8_output(y - e_y, scale, fmt)[0], fmt)
    hi = ofp8.decode(oe.fp8_output(y + e_y, scale, fmt)[0], fmt)
    d = ofp8.decode(np.asarray(codes, dtype=np.uint8), fmt)
    ok = (lo <= d) & (d <= hi)
    same = float(np.mean(np.asarray(codes) == oe.fp8_output(y, scale, fmt)[0]))
    print(f"[fused] {label} codes equal to the oracle's at its own value: {same:.5f}", flush=True)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{label}: {int((~ok).sum())} codes outside the interval; first {i}: gpu={d[i]} "
                             f"interval=[{lo[i]}, {hi[i]}] y={y[i]}")


def run_case(sq, mode, M, N, K, act, out, bias_kind, with_aux, seed, rows=None, amax0=0.0):
    label = f"{mode} {(M, N, K)} act{act} out{out} bias={bias_kind} aux={with_aux}"
    announce("fused gemm", label)
    rng = np.random.default_rng(seed)
    dev, orc, bmode = _operands(sq, rng, mode, M, N, K)
    bias = None if bias_kind is None else rng.standard_normal(N).astype(np.float32) * 0.5
    if bias is not None and bias_kind == "bf16":
        bias = ofp8.to_bf16(bias)
    bias_t = None if bias is None else _t(bias).to(torch.bfloat16 if bias_kind == "bf16" else torch.float32)
    aux_t = torch.empty((M, N), dtype=torch.bfloat16, device=DEV) if with_aux else None
    fmt = ofp8.E4M3 if out == E4 else ofp8.E5M2
    # a scale that makes the largest ~1% of outputs saturate
    cscale = np.float32(ofp8.FMAX[fmt] / 1.5) if out in (E4, E5) else np.float32(1)
    cs_t, amax_t = _scal(cscale), _scal(amax0)
    C = sq.fp8_gemm_fused(dev[0], 0, dev[1], dev[2], dev[3], 0, dev[4], dev[5], out_dtype=out, bias=bias_t, act=act,
                          aux=aux_t, c_scale=cs_t, c_amax=amax_t)
    torch.cuda.synchronize()
    r = np.arange(M) if rows is None else rows
    Cr, S, G = og.gemm_ref(orc[0], 0, orc[1], orc[2], orc[3], 0, orc[4], orc[5], rows=r)
    pre, y = oe.epilogue_ref(Cr, bias, act)
    e_pre = gemm_bound(S, G, K, bmode, False, Cr, Cr) + 2.0 ** -23 * (np.abs(pre) + 2.0 ** -10 * S)
    e_y = act_bound(pre, e_pre, act)
    got = np_of(C)[r]
    assert got.shape == y.shape, (got.shape, y.shape)
    if out in (F32, BF16):
        check_values(got, y, e_y, out == BF16, label)
    else:
        check_fp8(got, y, e_y, cscale, fmt, label)
        amax = float(np_of(amax_t)[0])
        lo_amax = max(amax0, float((np.abs(y) - e_y).max()))
        if rows is None:
            hi_amax = max(amax0, float((np.abs(y) + e_y).max()))
            assert lo_amax <= amax <= hi_amax * (1 + 2.0 ** -23), (label, amax, lo_amax, hi_amax)
        else:
            assert amax >= lo_amax, (label, amax, lo_amax)
    if with_aux:
        check_values(np_of(aux_t)[r], pre, e_pre, True, label + " aux")
    return C, amax_t


SMALL = [(200, 264, 256), (65, 130, 384), (1, 2, 128)]
COMBOS = [(NONE, F32, "f32", False), (GELU, BF16, "bf16", True), (SWIGLU, E4, "f32", True), (GELU, E5, None, False),
          (SWIGLU, BF16, None, False), (NONE, E4, "bf16", False)]


@pytest.mark.parametrize("combo", COMBOS)
@pytest.mark.parametrize("mnk", SMALL)
@pytest.mark.parametrize("mode", ["tensor", "block", "tile2", "mx"])
def test_fused_small(sq, mode, mnk, combo):
    act, out, bias_kind, with_aux = combo
    run_case(sq, mode, *mnk, act, out, bias_kind, with_aux, seed=sum(mnk) + 7 * act + 13 * out)


@pytest.mark.parametrize("act", [NONE, GELU])
def test_fused_odd_n(sq, act):
    """N odd: the unpaired store path of every kernel."""
    run_case(sq, "tensor", 33, 517, 256, act, BF16, "f32", True, seed=5)


# many tiles of the large-tile kernels (256 x 256 for tensor (at least 256 tiles) and MX,
# 256 x 128 blockwise); ragged M and N, N % 4 == 2 for the unaligned-quad paths (tensor and
# blockwise)
LARGE = {"tensor": (4100, 4102, 256), "mx": (2148, 4036, 384), "block": (2085, 3002, 384), "tile2": (1300, 4100, 256)}
LARGE_COMBOS = [(SWIGLU, E4, "bf16", True), (GELU, BF16, "f32", False), (NONE, E5, None, False),
                (SWIGLU, F32, "f32", False)]


@pytest.mark.parametrize("combo", LARGE_COMBOS)
@pytest.mark.parametrize("mode", ["tensor", "mx", "block", "tile2"])
def test_fused_large(sq, mode, combo):
    M, N, K = LARGE[mode]
    act, out, bias_kind, with_aux = combo
    rng = np.random.default_rng(M + N)
    r = np.sort(rng.choice(M, 160, replace=False))
    r[-1] = M - 1
    run_case(sq, mode, M, N, K, act, out, bias_kind, with_aux, seed=M + 3 * act + out, rows=r)


# blockwise problems whose 256 x 128 tiles leave at most 8 per XCD after the whole rounds (306
# and 272 tiles): the rest run as 256 x 64 halves in a second launch, fused epilogues included
LARGE_SPLIT = {"block": (2085, 4264, 256), "tile2": (2000, 4300, 256)}


@pytest.mark.parametrize("combo", LARGE_COMBOS[:3])
@pytest.mark.parametrize("mode", ["block", "tile2"])
def test_fused_split_launch(sq, mode, combo):
    M, N, K = LARGE_SPLIT[mode]
    act, out, bias_kind, with_aux = combo
    rng = np.random.default_rng(M + N + 1)
    r = np.sort(rng.choice(M, 160, replace=False))
    r[-1] = M - 1
    run_case(sq, mode, M, N, K, act, out, bias_kind, with_aux, seed=M + 5 * act + out, rows=r)


@pytest.mark.parametrize("mode", ["tensor", "mx", "block"])
def test_fused_plain_equals_fp8_gemm(sq, mode):
    """act NONE, no bias: the same fp32 values as fp8_gemm, bit for bit, and the FP8 output's
    amax is the largest |value| of that fp32 output exactly."""
    M, N, K = LARGE[mode] if mode != "block" else (2085, 3004, 384)
    announce("fused plain == fp8_gemm", mode)
    rng = np.random.default_rng(11)
    dev, _, _ = _operands(sq, rng, mode, M, N, K)
    C0 = sq.fp8_gemm(dev[0], 0, dev[1], dev[2], dev[3], 0, dev[4], dev[5], sq.OUT_F32)
    C1 = sq.fp8_gemm_fused(dev[0], 0, dev[1], dev[2], dev[3], 0, dev[4], dev[5], out_dtype=sq.OUT_F32)
    amax = _scal(0.0)
    sq.fp8_gemm_fused(dev[0], 0, dev[1], dev[2], dev[3], 0, dev[4], dev[5], out_dtype=sq.OUT_E4M3,
                      c_scale=_scal(1.0), c_amax=amax)
    torch.cuda.synchronize()
    assert torch.equal(C0, C1)
    assert amax.item() == C0.abs().max().item()


def test_amax_accumulates(sq):
    """The output amax is max-reduced into the slot: a larger prior value stays."""
    run_case(sq, "tensor", 200, 264, 256, GELU, E4, "f32", False, seed=3, amax0=1e6)


def test_fused_argument_errors(sq):
    A = torch.zeros((4, 128), dtype=torch.uint8, device=DEV)
    B = torch.zeros((6, 128), dtype=torch.uint8, device=DEV)
    B5 = torch.zeros((5, 128), dtype=torch.uint8, device=DEV)
    one = _scal(1.0)
    with pytest.raises(sq.Fp8Error) as e:
        # the binding takes C as [M][N // 2]; the library rejects the odd N
        sq.fp8_gemm_fused(A, 0, one, 0, B5, 0, one, 0, out_dtype=sq.OUT_F32, act=sq.FP8_ACT_SWIGLU,
                          C=torch.empty((4, 2), device=DEV))
    assert e.value.code == sq.FP8_ERR_SHAPE
    with pytest.raises(sq.Fp8Error) as e:
        sq.fp8_gemm_fused(A, 0, one, 0, B, 0, one, 0, out_dtype=sq.OUT_E4M3)  # no c_scale / c_amax
    assert e.value.code == sq.FP8_ERR_ARG
    with pytest.raises(sq.Fp8Error) as e:
        sq.fp8_gemm_fused(A, 0, one, 0, B, 0, one, 0, out_dtype=sq.OUT_F32, act=7)
    assert e.value.code == sq.FP8_ERR_ARG


def test_workload4_fc1_swiglu_to_fp8(sq):
    """X [8192x4096] x W [14336x4096] (gate/up interleaved), per-tensor delayed scales, SwiGLU
    fused, E4M3 output for the down projection with its amax in a recipe slot; sampled rows."""
    import workloads

    announce("workload4 fused SwiGLU fc1")
    X, W, _ = workloads.w4_inputs()
    ox, ow = X.float().numpy(), W.float().numpy()
    E4M3 = ofp8.E4M3
    sx = np.float32(448.0 / np.abs(ox).max())
    sw = np.float32(448.0 / np.abs(ow).max())
    Xd, Wd = X.to(DEV), W.to(DEV)
    qx, _ = sq.fp8_quantize(Xd, E4M3, sq.FP8_SCALE_TENSOR, scale=_scal(sx))
    qw, _ = sq.fp8_quantize(Wd, E4M3, sq.FP8_SCALE_TENSOR, scale=_scal(sw))
    sa, sb = np.float32(1) / sx, np.float32(1) / sw
    cscale = np.float32(448.0 / 2.0)
    amax = _scal(0.0)
    H = sq.fp8_gemm_fused(qx, E4M3, _scal(sa), 0, qw, E4M3, _scal(sb), 0, out_dtype=sq.OUT_E4M3,
                          act=sq.FP8_ACT_SWIGLU, c_scale=_scal(cscale), c_amax=amax)
    torch.cuda.synchronize()
    assert tuple(H.shape) == (8192, 7168)
    rng = np.random.default_rng(44)
    r = np.sort(rng.choice(8192, 24, replace=False))
    oqx_r = oq.quantize_tensor(ox[r], sx, E4M3)[0]
    oqw = oq.quantize_tensor(ow, sw, E4M3)[0]
    Cr, S, G = og.gemm_ref(oqx_r, E4M3, sa, og.TENSOR, oqw, E4M3, sb, og.TENSOR)
    pre, y = oe.epilogue_ref(Cr, None, SWIGLU)
    e_pre = gemm_bound(S, G, 4096, "tensor", False, Cr, Cr)
    e_y = act_bound(pre, e_pre, SWIGLU)
    check_fp8(np_of(H[torch.from_numpy(r).to(DEV)]), y, e_y, cscale, E4M3, "workload4 fused fc1")
    assert amax.item() >= float((np.abs(y) - e_y).max())


@pytest.mark.parametrize("act", [NONE, GELU, SWIGLU])
def test_fused_k_zero_is_the_activation_of_the_bias(sq, act):
    """K = 0: the GEMM part is exactly 0, so the output is act(bias) (act(0) without bias)."""
    announce("fused K = 0", act)
    M, N = 70, 258
    A = torch.empty((M, 0), dtype=torch.uint8, device=DEV)
    B = torch.empty((N, 0), dtype=torch.uint8, device=DEV)
    bias = np.linspace(-4, 4, N).astype(np.float32)
    C = sq.fp8_gemm_fused(A, 0, _scal(1.0), 0, B, 0, _scal(1.0), 0, out_dtype=sq.OUT_F32, bias=_t(bias), act=act)
    torch.cuda.synchronize()
    pre, y = oe.epilogue_ref(np.zeros((M, N)), bias, act)
    e = act_bound(pre, np.zeros_like(pre), act)
    check_values(np_of(C), y, e, False, f"K=0 act{act}")


def test_fp8_weight_stored_once(sq):
    """Quantize-once FP8 weights (the tutorial's fp8_model_init idea): the weight's codes and
    scale_inv are made once and reused by every step's GEMM, with fresh activations each step;
    each step equals the oracle on the stored codes."""
    import workloads

    W = workloads.w1_weight()
    sw = np.float32(448.0 / float(W.abs().max()))
    qw, _ = sq.fp8_quantize(W.to(DEV), 0, sq.FP8_SCALE_TENSOR, scale=_scal(sw))
    torch.cuda.synchronize()
    stored = np_of(qw).copy()
    for step in range(3):
        announce("stored FP8 weight, step", step)
        X = workloads.w1_input(step)
        sx = np.float32(448.0 / float(X.abs().max()))
        qx, _ = sq.fp8_quantize(X.to(DEV), 0, sq.FP8_SCALE_TENSOR, scale=_scal(sx))
        Y = sq.fp8_gemm_fused(qx, 0, _scal(np.float32(1) / sx), 0, qw, 0, _scal(np.float32(1) / sw), 0,
                              out_dtype=sq.OUT_F32)
        torch.cuda.synchronize()
        assert np.array_equal(np_of(qw), stored), "stored weight codes changed"
        oqx = oq.quantize_tensor(X.numpy(), sx, 0)[0]
        oqw = oq.quantize_tensor(W.numpy(), sw, 0)[0]
        assert np.array_equal(stored, oqw)
        Cr, S, G = og.gemm_ref(oqx, 0, np.float32(1) / sx, og.TENSOR, oqw, 0, np.float32(1) / sw, og.TENSOR)
        check_values(np_of(Y), Cr, gemm_bound(S, G, 256, "tensor", False, Cr, Cr), False, f"stored W step {step}")


def _random_cases(n=32, seed=2024):
    """Seeded random shapes over every kernel path: M, N from 1 to 1100 (ragged, odd, tiny),
    K a multiple of 128 up to 1024, every mode, activation, output type and bias type."""
    rng = np.random.default_rng(seed)
    modes = ["tensor", "mx", "block", "tile2"]
    out = []
    for i in range(n):
        mode = modes[i % 4]
        M = int(rng.integers(1, 1101))
        N = int(rng.integers(1, 1101))
        act = int(rng.integers(0, 3))
        if act == SWIGLU:
            N += N % 2
        if mode == "mx" and rng.random() < 0.5:  # half the MX cases on the 256x256 kernel
            M, N = M + (-M) % 4, N + (-N) % 4
        K = 128 * int(rng.integers(1, 9))
        o = int(rng.integers(0, 4))
        bias_kind = [None, "f32", "bf16"][int(rng.integers(0, 3))]
        out.append((mode, M, N, K, act, o, bias_kind, bool(rng.random() < 0.3), 1000 + i))
    return out


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-a{c[4]}o{c[5]}")
def test_fused_random_shapes(sq, case):
    mode, M, N, K, act, out, bias_kind, with_aux, seed = case
    run_case(sq, mode, M, N, K, act, out, bias_kind, with_aux, seed=seed)
