"""FP8 weight storage (quantise once, reuse): the weight is cast to E4M3 one time with the
current per-tensor scale of its own amax, and its codes and scale_inv are kept; every later
step quantises only its new activations (delayed scaling) and calls fp8_gemm with the stored
weight.  This is the inference form the Transformer Engine tutorial's closing list of
extensions names (weights kept in FP8 for inference), built from the existing entry points.  Each step's codes, recipe state and GEMM output
match the oracle; the stored codes are never rewritten."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import (DEV, announce, assert_codes_equal, assert_f32_bits_equal, check_gemm, f32_np,  # noqa: E402
                      np_of)
from oracle import fp8 as ofp8, gemm as og, quantize as oq, recipe as orc  # noqa: E402


def test_weight_quantised_once_and_reused():
    import scaled_quantize_gemm_amd as sq
    import workloads

    E4 = ofp8.E4M3
    N, K, M, steps = 768, 1024, 512, 4
    announce("weight storage: quantise W once", (N, K))
    W = workloads.normal((N, K), 0.02, 7, 900, torch.bfloat16)
    w_np = f32_np(W)
    s_w, si_w = (np.float32(v) for v in orc.current_scale(np.float32(np.abs(w_np).max()), E4))
    qW, _ = sq.fp8_quantize(W.to(DEV), E4, sq.FP8_SCALE_TENSOR,
                            scale=torch.tensor([float(s_w)], dtype=torch.float32, device=DEV))
    stored = qW.clone()
    assert_codes_equal(np_of(qW), oq.quantize_tensor(w_np, s_w, E4)[0], "stored W codes")
    w_scale_inv = torch.tensor([float(si_w)], dtype=torch.float32, device=DEV)

    st = sq.DelayedScalingState([E4], history_len=16, device=DEV)
    ost = orc.DelayedState(1, 16)
    for t in range(steps):
        announce("weight storage: step", t)
        X = workloads.normal((M, K), 1.0 + 0.5 * t, 7, 901 + t, torch.bfloat16)
        scale, slot, scale_inv = st.slot(0)
        qx, _ = sq.fp8_quantize(X.to(DEV), E4, sq.FP8_SCALE_TENSOR, scale=scale, amax_slot=slot)
        Y = sq.fp8_gemm(qx, E4, scale_inv, 0, qW, E4, w_scale_inv, 0, sq.OUT_BF16)
        torch.cuda.synchronize()
        x_np = f32_np(X)
        oqx, oax = oq.quantize_tensor(x_np, ost.scale[0], E4)
        assert_codes_equal(np_of(qx), oqx, f"X codes step {t}")
        C, S, G = og.gemm_ref(oqx, E4, ost.scale_inv[0], 0, oq.quantize_tensor(w_np, s_w, E4)[0], E4, si_w, 0)
        check_gemm(np_of(Y), C, S, G, K, "tensor", True, f"step {t}")
        ost.record(0, oax)
        st.update()
        ost = orc.delayed_update(ost, [E4])
        torch.cuda.synchronize()
        assert_f32_bits_equal(np_of(st.scale), ost.scale, f"scale after step {t}")
        assert torch.equal(qW, stored), f"stored weight codes changed at step {t}"
