"""GPU parity of the delayed-scaling recipe: workload 1 end to end, checkpoint/resume, edge cases."""

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


def _step(sq, st, X, W):
    sx, ax, six = st.slot(0)
    sw, aw, siw = st.slot(1)
    qx, _ = sq.fp8_quantize(X, sq.FP8_E4M3, sq.FP8_SCALE_TENSOR, scale=sx, amax_slot=ax)
    qw, _ = sq.fp8_quantize(W, sq.FP8_E4M3, sq.FP8_SCALE_TENSOR, scale=sw, amax_slot=aw)
    Y = sq.fp8_gemm(qx, sq.FP8_E4M3, six, sq.FP8_SCALE_TENSOR, qw, sq.FP8_E4M3, siw, sq.FP8_SCALE_TENSOR, sq.OUT_F32)
    return qx, qw, Y


def test_workload1_sixteen_steps(sq):
    """Per-tensor delayed scaling, HYBRID forward (E4M3 X, W), history 16, max, margin 0; seed 0."""
    import workloads

    st = sq.DelayedScalingState([sq.FP8_E4M3, sq.FP8_E4M3], history_len=16, device=DEV)
    ost = orc.DelayedState(2, 16)
    W = workloads.w1_weight()
    Wd = W.to(DEV)
    for step in range(16):
        announce("workload1 step", step)
        X = workloads.w1_input(step)
        qx, qw, Y = _step(sq, st, X.to(DEV), Wd)
        torch.cuda.synchronize()
        oqx, oax = oq.quantize_tensor(X.numpy(), ost.scale[0], ofp8.E4M3)
        oqw, oaw = oq.quantize_tensor(W.numpy(), ost.scale[1], ofp8.E4M3)
        assert_codes_equal(np_of(qx), oqx, f"X step {step}")
        assert_codes_equal(np_of(qw), oqw, f"W step {step}")
        ost.record(0, oax)
        ost.record(1, oaw)
        assert_f32_bits_equal(np_of(st.amax_history), ost.hist, f"history after casts, step {step}")
        C, S, G = og.gemm_ref(oqx, ofp8.E4M3, ost.scale_inv[0], og.TENSOR, oqw, ofp8.E4M3, ost.scale_inv[1], og.TENSOR)
        check_gemm(np_of(Y), C, S, G, 256, "tensor", False, f"workload1 step {step}")
        st.update()
        ost = orc.delayed_update(ost, [ofp8.E4M3, ofp8.E4M3])
        torch.cuda.synchronize()
        assert_f32_bits_equal(np_of(st.scale), ost.scale, f"scale step {step}")
        assert_f32_bits_equal(np_of(st.scale_inv), ost.scale_inv, f"scale_inv step {step}")
        assert_f32_bits_equal(np_of(st.amax_history), ost.hist, f"rolled history step {step}")
    # readback in the tutorial's shape: scale[:4], amax_history[0, :4]
    assert st.scale.flatten()[:4].tolist() == [float(v) for v in ost.scale[:4]]


def test_checkpoint_resume_is_byte_identical(sq):
    import workloads

    announce("checkpoint / resume")
    W = workloads.w1_weight().to(DEV)

    def run(st, steps):
        outs = []
        for t in steps:
            qx, qw, Y = _step(sq, st, workloads.w1_input(t).to(DEV), W)
            st.update()
            outs.append((np_of(qx), np_of(Y)))
        return outs

    a = sq.DelayedScalingState([0, 0], device=DEV)
    straight = run(a, range(16))
    b = sq.DelayedScalingState([0, 0], device=DEV)
    first = run(b, range(8))
    saved = {k: getattr(b, k).cpu().clone() for k in ("amax_history", "scale", "scale_inv")}
    c = sq.DelayedScalingState([0, 0], device=DEV)
    for k, v in saved.items():
        getattr(c, k).copy_(v.to(DEV))
    second = run(c, range(8, 16))
    torch.cuda.synchronize()
    for (q1, y1), (q2, y2) in zip(straight, first + second):
        assert np.array_equal(q1, q2) and np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(np_of(a.scale), np_of(c.scale))


@pytest.mark.parametrize("H,n", [(1, 3), (16, 5), (1024, 2), (4, 5000)])
def test_recipe_update_edge_cases(sq, H, n):
    announce("recipe update", H, n)
    rng = np.random.default_rng(H * 7 + n)
    hist = rng.uniform(0, 50, (H, n)).astype(np.float32)
    hist[:, 0] = 0.0  # zero window: keep
    if n > 2:
        hist[H // 2, 1] = np.nan  # NaN in window: keep
        hist[0, 2] = np.inf  # inf: keep
    if n > 4:
        hist[:, 4] = 1e-40  # tiny: fmax/m overflows -> FLT_MAX
    fmts = [int(v) for v in rng.integers(0, 2, n)]
    scale0 = rng.uniform(0.5, 2, n).astype(np.float32)
    for margin in (0, 3):
        ost = orc.DelayedState(n, H)
        ost.hist[...] = hist
        ost.scale[...] = scale0
        ost.scale_inv[...] = np.float32(1) / scale0
        st = sq.DelayedScalingState(fmts, history_len=H, margin=margin, device=DEV)
        st.amax_history.copy_(torch.from_numpy(hist))
        st.scale.copy_(torch.from_numpy(scale0))
        st.scale_inv.copy_(torch.from_numpy(np.float32(1) / scale0))
        st.update()
        ost = orc.delayed_update(ost, fmts, margin)
        torch.cuda.synchronize()
        assert_f32_bits_equal(np_of(st.scale), ost.scale, "scale")
        assert_f32_bits_equal(np_of(st.scale_inv), ost.scale_inv, "scale_inv")
        assert_f32_bits_equal(np_of(st.amax_history), ost.hist, "history")


def test_determinism(sq):
    import workloads

    announce("determinism")
    x = workloads.w4_inputs(m=1024, k=4096, n=256)[0].to(DEV)
    outs = []
    for _ in range(2):
        s = torch.tensor([40.0], device=DEV)
        slot = torch.zeros(1, device=DEV)
        q, qT = sq.fp8_cast_transpose(x, sq.FP8_E4M3, s, amax_slot=slot)
        si = torch.tensor([0.025], device=DEV)
        Y = sq.fp8_gemm(q, 0, si, 0, q[:256].contiguous(), 0, si, 0, sq.OUT_BF16)
        torch.cuda.synchronize()
        outs.append((np_of(q), np_of(qT), np_of(slot), np_of(Y)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
