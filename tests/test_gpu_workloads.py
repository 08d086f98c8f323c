"""The five workloads at full size, launched as the bench launches them; the oracle checks
sampled rows / columns (codes and scales bit-exact, GEMM within the derived bound)."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import DEV, announce, assert_codes_equal, assert_f32_bits_equal, check_gemm, f32_np, np_of  # noqa
from oracle import fp8 as ofp8, gemm as og, quantize as oq, recipe as orc  # noqa: E402


@pytest.fixture(scope="module")
def sq():
    import scaled_quantize_gemm_amd as m

    return m


def _idx(rng, n, k):
    return np.sort(rng.choice(n, min(k, n), replace=False))


def _rows(t, idx):
    return np_of(t[torch.from_numpy(idx).to(t.device)])


def _scal(v):
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def test_workload2_minigpt_layer_set(sq):
    """Forward E4M3 x E4M3, dgrad / wgrad E5M2 x E4M3, cast-transposes, delayed recipe, 2 steps."""
    import workloads

    E4, E5 = ofp8.E4M3, ofp8.E5M2
    fmts = []
    for _ in workloads.MINIGPT_LAYERS:
        fmts += [E4, E4, E5]  # X, W, dY slots per layer
    st = sq.DelayedScalingState(fmts, history_len=16, device=DEV)
    ost = orc.DelayedState(len(fmts), 16)
    rng = np.random.default_rng(2)
    for step in range(2):
        for li, (name, k_in, n_out) in enumerate(workloads.MINIGPT_LAYERS):
            announce("workload2", name, "step", step)
            X, W, dY = workloads.w2_layer(li, step)
            sl = [3 * li, 3 * li + 1, 3 * li + 2]
            views = [st.slot(j) for j in sl]
            qx, qxT = sq.fp8_cast_transpose(X.to(DEV), E4, views[0][0], amax_slot=views[0][1])
            qw, qwT = sq.fp8_cast_transpose(W.to(DEV), E4, views[1][0], amax_slot=views[1][1])
            qd, qdT = sq.fp8_cast_transpose(dY.to(DEV), E5, views[2][0], amax_slot=views[2][1])
            Y = sq.fp8_gemm(qx, E4, views[0][2], 0, qw, E4, views[1][2], 0, sq.OUT_BF16)
            dX = sq.fp8_gemm(qd, E5, views[2][2], 0, qwT, E4, views[1][2], 0, sq.OUT_BF16)
            dW = sq.fp8_gemm(qdT, E5, views[2][2], 0, qxT, E4, views[0][2], 0, sq.OUT_BF16)
            torch.cuda.synchronize()
            ox, ow, od = f32_np(X), f32_np(W), f32_np(dY)
            oqx, oqxT, oax = oq.cast_transpose(ox, ost.scale[sl[0]], E4)
            oqw, oqwT, oaw = oq.cast_transpose(ow, ost.scale[sl[1]], E4)
            oqd, oqdT, oad = oq.cast_transpose(od, ost.scale[sl[2]], E5)
            for got, want, nm in ((qx, oqx, "X"), (qxT, oqxT, "XT"), (qw, oqw, "W"), (qwT, oqwT, "WT"),
                                  (qd, oqd, "dY"), (qdT, oqdT, "dYT")):
                assert_codes_equal(np_of(got), want, f"{name} {nm} step {step}")
            for j, a in zip(sl, (oax, oaw, oad)):
                ost.record(j, a)
            si = ost.scale_inv
            r = _idx(rng, 2048, 96)
            C, S, G = og.gemm_ref(oqx, E4, si[sl[0]], 0, oqw, E4, si[sl[1]], 0, rows=r)
            check_gemm(_rows(Y, r), C, S, G, k_in, "tensor", True, f"{name} fwd")
            C, S, G = og.gemm_ref(oqd, E5, si[sl[2]], 0, oqwT, E4, si[sl[1]], 0, rows=r)
            check_gemm(_rows(dX, r), C, S, G, n_out, "tensor", True, f"{name} dgrad")
            r2 = _idx(rng, n_out, 96)
            C, S, G = og.gemm_ref(oqdT, E5, si[sl[2]], 0, oqxT, E4, si[sl[0]], 0, rows=r2)
            check_gemm(_rows(dW, r2), C, S, G, 2048, "tensor", True, f"{name} wgrad")
        assert_f32_bits_equal(np_of(st.amax_history), ost.hist, f"history step {step}")
        st.update()
        ost = orc.delayed_update(ost, fmts)
        torch.cuda.synchronize()
        assert_f32_bits_equal(np_of(st.scale), ost.scale, f"scales step {step}")
        assert_f32_bits_equal(np_of(st.scale_inv), ost.scale_inv, f"scale_inv step {step}")


def test_workload3_blockwise(sq):
    """X [4096x7168] 1x128 tiles (0.1% outliers x100), W [7168x7168] 128x128 blocks, bf16 out."""
    import workloads

    announce("workload3 blockwise full size")
    X, W = workloads.w3_inputs()
    qx, sx = sq.fp8_quantize(X.to(DEV), 0, sq.FP8_SCALE_TILE_1x128)
    qw, sw = sq.fp8_quantize(W.to(DEV), 0, sq.FP8_SCALE_BLOCK_128x128)
    Y = sq.fp8_gemm(qx, 0, sx, sq.FP8_SCALE_TILE_1x128, qw, 0, sw, sq.FP8_SCALE_BLOCK_128x128, sq.OUT_BF16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    r = _idx(rng, 4096, 64)
    ox = f32_np(X)[r]
    oqx, osx = oq.quantize_tile_1x128(ox, 0)
    assert_codes_equal(_rows(qx, r), oqx, "X tiles")
    assert_f32_bits_equal(np_of(sx)[:, r], osx, "X tile scale_inv")
    ow = f32_np(W)
    oqw, osw = oq.quantize_block_128x128(ow, 0)
    assert_codes_equal(np_of(qw), oqw, "W blocks")
    assert_f32_bits_equal(np_of(sw), osw, "W block scale_inv")
    # oracle-only operands for the sampled rows (other rows are never read by the check)
    qx_s = np.zeros((4096, 7168), np.uint8)
    qx_s[r] = oqx
    sx_s = np.ones((56, 4096), np.float32)
    sx_s[:, r] = osx
    C, S, G = og.gemm_ref(qx_s, 0, sx_s, og.TILE_1x128, oqw, 0, osw, og.BLOCK_128x128, rows=r)
    check_gemm(_rows(Y, r), C, S, G, 7168, "block", True, "workload3 GEMM")


def test_workload4_fc1_fwd_bwd(sq):
    """X [8192x4096], W [14336x4096], dY [8192x14336]; fwd, dgrad, wgrad; delayed scaling, 2 steps."""
    import workloads

    E4, E5 = ofp8.E4M3, ofp8.E5M2
    X, W, dY = workloads.w4_inputs()
    Xd, Wd, dYd = X.to(DEV), W.to(DEV), dY.to(DEV)
    st = sq.DelayedScalingState([E4, E4, E5], device=DEV)
    ox, ow, od = f32_np(X), f32_np(W), f32_np(dY)
    ost = orc.DelayedState(3, 16)  # the oracle's own recipe state, stepped alongside
    for j, x in enumerate((ox, ow, od)):
        ost.record(j, orc.amax(x))
    ost1 = orc.delayed_update(ost, [E4, E4, E5])
    for step in range(2):
        announce("workload4 step", step)
        sc = [st.slot(j) for j in range(3)]
        qx, qxT = sq.fp8_cast_transpose(Xd, E4, sc[0][0], amax_slot=sc[0][1])
        qw, _ = sq.fp8_quantize(Wd, E4, sq.FP8_SCALE_TENSOR, scale=sc[1][0], amax_slot=sc[1][1])
        _, qwT = sq.fp8_cast_transpose(Wd, E4, sc[1][0])
        qd, qdT = sq.fp8_cast_transpose(dYd, E5, sc[2][0], amax_slot=sc[2][1])
        Y = sq.fp8_gemm(qx, E4, sc[0][2], 0, qw, E4, sc[1][2], 0, sq.OUT_BF16)
        dX = sq.fp8_gemm(qd, E5, sc[2][2], 0, qwT, E4, sc[1][2], 0, sq.OUT_BF16)
        dW = sq.fp8_gemm(qdT, E5, sc[2][2], 0, qxT, E4, sc[0][2], 0, sq.OUT_BF16)
        torch.cuda.synchronize()
        if step == 1:
            assert_f32_bits_equal(np_of(st.scale), ost1.scale, "step-1 scales")
            s, si = ost1.scale, ost1.scale_inv
            rng = np.random.default_rng(4)
            announce("workload4 oracle: X, W codes")
            oqx = oq.quantize_tensor(ox, s[0], E4)[0]
            oqw = oq.quantize_tensor(ow, s[1], E4)[0]
            assert_codes_equal(np_of(qx), oqx, "X")
            assert_codes_equal(np_of(qw), oqw, "W")
            r = _idx(rng, 8192, 32)
            r2 = _idx(rng, 14336, 24)
            oqd_r = oq.quantize_tensor(od[r], s[2], E5)[0]
            oqd_c = oq.quantize_tensor(np.ascontiguousarray(od[:, r2].T), s[2], E5)[0]
            assert_codes_equal(_rows(qd, r), oqd_r, "dY rows")
            assert_codes_equal(_rows(qdT, r2), oqd_c, "dY^T rows")
            announce("workload4 oracle: fwd")
            C, S, G = og.gemm_ref(oqx, E4, si[0], 0, oqw, E4, si[1], 0, rows=r)
            check_gemm(_rows(Y, r), C, S, G, 4096, "tensor", True, "workload4 fwd")
            announce("workload4 oracle: dgrad")
            C, S, G = og.gemm_ref(oqd_r, E5, si[2], 0, np.ascontiguousarray(oqw.T), E4, si[1], 0)
            check_gemm(_rows(dX, r), C, S, G, 14336, "tensor", True, "workload4 dgrad")
            announce("workload4 oracle: wgrad")
            C, S, G = og.gemm_ref(oqd_c, E5, si[2], 0, np.ascontiguousarray(oqx.T), E4, si[0], 0)
            check_gemm(_rows(dW, r2), C, S, G, 8192, "tensor", True, "workload4 wgrad")
        st.update()


def test_workload5_mx_and_stream(sq):
    """MX E4M3 8192^3 GEMM (bf16 out) and the 2^28-element amax + cast stream."""
    import workloads

    announce("workload5 MX full size")
    A, B = workloads.w5_inputs()
    qa, ea = sq.fp8_quantize(A.to(DEV), 0, sq.FP8_SCALE_MX_1x32)
    qb, eb = sq.fp8_quantize(B.to(DEV), 0, sq.FP8_SCALE_MX_1x32)
    C = sq.fp8_gemm(qa, 0, ea, sq.FP8_SCALE_MX_1x32, qb, 0, eb, sq.FP8_SCALE_MX_1x32, sq.OUT_BF16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    r = _idx(rng, 8192, 32)
    oqa, oea = oq.quantize_mx_1x32(f32_np(A[torch.from_numpy(r)]), 0)
    assert_codes_equal(_rows(qa, r), oqa, "A codes")
    assert_codes_equal(np_of(ea)[:, r].T, oea, "A e8m0")
    oqb, oeb = oq.quantize_mx_1x32(f32_np(B), 0)
    assert_codes_equal(np_of(qb), oqb, "B codes")
    assert_codes_equal(np_of(eb).T, oeb, "B e8m0")
    Cr, S, G = og.gemm_ref(oqa, 0, oea, og.MX_1x32, oqb, 0, oeb, og.MX_1x32)
    check_gemm(_rows(C, r), Cr, S, G, 8192, "mx", True, "workload5 MX GEMM")
    del A, B, qa, qb, C
    announce("workload5 stream 2^28 amax + cast")
    T = workloads.w5_stream()
    s = _scal(np.float32(448.0) / np.float32(5.5))
    slot = torch.zeros(1, device=DEV)
    q, _ = sq.fp8_quantize(T.to(DEV), 0, sq.FP8_SCALE_TENSOR, scale=s, amax_slot=slot)
    torch.cuda.synchronize()
    t = f32_np(T)
    assert_f32_bits_equal(np_of(slot), [np.abs(t).max()], "stream amax")
    for start in (0, (1 << 27) + 12345, (1 << 28) - 4096):
        seg = slice(start, start + 4096)
        assert_codes_equal(np_of(q[seg]), oq.quantize_tensor(t[seg], np.float32(s.item()), 0)[0], f"stream @{start}")
