"""The five workloads at full size, launched as the bench launches them.

Codes, scales, amax history and e8m0 bytes are compared with the oracle bit for bit over
whole tensors (the oracle's elementwise quantisers run in threads over row chunks); GEMM
outputs are checked on sampled rows against the oracle within the derived bound (with the
fraction inside the stated 2^-18 S recorded) and bit for bit against the matrix-core model.
Workloads 2 and 4 run 20+ delayed-scaling steps with an amax spike that must enter the
scales for exactly the history length and then age out.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import mfma_model as mm  # noqa: E402
from gpu_util import (DEV, announce, assert_codes_equal, assert_f32_bits_equal, check_gemm, f32_np, np_of,  # noqa
                      par_rows)
from oracle import fp8 as ofp8, gemm as og, quantize as oq, recipe as orc  # noqa: E402

E4, E5 = ofp8.E4M3, ofp8.E5M2
H = 16


@pytest.fixture(scope="module")
def sq():
    import scaled_quantize_gemm_amd as m

    return m


def _idx(rng, n, k):
    r = np.sort(rng.choice(n, min(k, n), replace=False))
    r[0], r[-1] = 0, n - 1
    return np.unique(r)


def _rows(t, idx):
    return np_of(t[torch.from_numpy(idx).to(t.device)])


def _scal(v):
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def _cast_transpose(x, scale, fmt):
    """oracle cast_transpose over row chunks in threads -> (q, qT, amax)."""
    parts = par_rows(oq.quantize_tensor, x, np.float32(scale), fmt)
    q = np.concatenate([p[0] for p in parts])
    return q, np.ascontiguousarray(q.T), np.float32(np.max(np.array([p[1] for p in parts], np.float32)))


def _model_rows(C, A, fa, sa, B, fb, sb, rows, label, out_bf16=True):
    """GPU rows equal the matrix-core model bit for bit (bf16: the RNE of its fp32)."""
    em = mm.emulate_gemm(A, fa, np.float32(sa), mm.TENSOR, B, fb, np.float32(sb), mm.TENSOR, rows=rows,
                         out_bf16=out_bf16)
    got = _rows(C, rows).astype(np.float64)
    bad = got != em
    assert not bad.any(), f"{label}: {int(bad.sum())} outputs differ from the matrix-core model"


SPIKE2 = 4
STEPS2 = SPIKE2 + H + 2


def test_workload2_minigpt_layer_set(sq):
    """MiniGPT layer set, delayed scaling (HYBRID: E4M3 X and W, E5M2 dY), 22 steps; at step 4
    layer 0's X is 8x larger.  Codes of q and qT, the history and the scales are compared
    every step; GEMMs (fwd, dgrad, wgrad) at the first and the last step."""
    import workloads

    fmts = []
    for _ in workloads.MINIGPT_LAYERS:
        fmts += [E4, E4, E5]  # X, W, dY slots per layer
    n = len(fmts)
    st = sq.DelayedScalingState(fmts, history_len=H, device=DEV)
    ost = orc.DelayedState(n, H)
    rng = np.random.default_rng(2)
    scale0 = []
    for step in range(STEPS2):
        announce("workload2 step", step)
        ins = [workloads.w2_layer(li, step) for li in range(len(workloads.MINIGPT_LAYERS))]
        if step == SPIKE2:
            X, W, dY = ins[0]
            ins[0] = (X * 8, W, dY)  # a power of two: exact in bf16
        gpu = []
        for li, (X, W, dY) in enumerate(ins):
            sl = [3 * li + j for j in range(3)]
            v = [st.slot(j) for j in sl]
            qx, qxT = sq.fp8_cast_transpose(X.to(DEV), E4, v[0][0], amax_slot=v[0][1])
            qw, qwT = sq.fp8_cast_transpose(W.to(DEV), E4, v[1][0], amax_slot=v[1][1])
            qd, qdT = sq.fp8_cast_transpose(dY.to(DEV), E5, v[2][0], amax_slot=v[2][1])
            Y = sq.fp8_gemm(qx, E4, v[0][2], 0, qw, E4, v[1][2], 0, sq.OUT_BF16)
            dX = sq.fp8_gemm(qd, E5, v[2][2], 0, qwT, E4, v[1][2], 0, sq.OUT_BF16)
            dW = sq.fp8_gemm(qdT, E5, v[2][2], 0, qxT, E4, v[0][2], 0, sq.OUT_BF16)
            gpu.append(((qx, qxT), (qw, qwT), (qd, qdT), Y, dX, dW))
        torch.cuda.synchronize()
        si = ost.scale_inv.copy()
        for li, ((X, W, dY), g) in enumerate(zip(ins, gpu)):
            name, k_in, n_out = workloads.MINIGPT_LAYERS[li]
            sl = [3 * li + j for j in range(3)]
            o = [_cast_transpose(f32_np(t), ost.scale[j], f) for t, j, f in zip((X, W, dY), sl, (E4, E4, E5))]
            for (gq, gqT), (oq_, oqT, _), nm in zip(g[:3], o, ("X", "W", "dY")):
                assert_codes_equal(np_of(gq), oq_, f"{name} {nm} step {step}")
                assert_codes_equal(np_of(gqT), oqT, f"{name} {nm}^T step {step}")
            for j, (_, _, a) in zip(sl, o):
                ost.record(j, a)
            if step in (0, STEPS2 - 1):
                Y, dX, dW = g[3:]
                (oqx, oqxT, _), (oqw, oqwT, _), (oqd, oqdT, _) = o
                r = _idx(rng, 2048, 64)
                C, S, G = og.gemm_ref(oqx[r], E4, si[sl[0]], 0, oqw, E4, si[sl[1]], 0)
                check_gemm(_rows(Y, r), C, S, G, k_in, "tensor", True, f"workload2 {name} fwd step {step}")
                C, S, G = og.gemm_ref(oqd[r], E5, si[sl[2]], 0, oqwT, E4, si[sl[1]], 0)
                check_gemm(_rows(dX, r), C, S, G, n_out, "tensor", True, f"workload2 {name} dgrad step {step}")
                r2 = _idx(rng, n_out, 64)
                C, S, G = og.gemm_ref(oqdT[r2], E5, si[sl[2]], 0, oqxT, E4, si[sl[0]], 0)
                check_gemm(_rows(dW, r2), C, S, G, 2048, "tensor", True, f"workload2 {name} wgrad step {step}")
                _model_rows(Y, oqx, E4, si[sl[0]], oqw, E4, si[sl[1]], r[:4], f"{name} fwd model")
                _model_rows(dX, oqd, E5, si[sl[2]], oqwT, E4, si[sl[1]], r[:4], f"{name} dgrad model")
                _model_rows(dW, oqdT, E5, si[sl[2]], oqxT, E4, si[sl[0]], r2[:4], f"{name} wgrad model")
        assert_f32_bits_equal(np_of(st.amax_history), ost.hist, f"history step {step}")
        st.update()
        ost = orc.delayed_update(ost, fmts)
        torch.cuda.synchronize()
        assert_f32_bits_equal(np_of(st.scale), ost.scale, f"scales after step {step}")
        assert_f32_bits_equal(np_of(st.scale_inv), ost.scale_inv, f"scale_inv after step {step}")
        assert_f32_bits_equal(np_of(st.amax_history), ost.hist, f"rolled history after step {step}")
        scale0.append(float(ost.scale[0]))
    # the spike sets layer 0's X scale for exactly H steps, then ages out
    spike = scale0[SPIKE2]
    assert all(s == spike for s in scale0[SPIKE2:SPIKE2 + H]), scale0
    assert scale0[SPIKE2 + H] > spike and scale0[SPIKE2 - 1] > spike


def test_workload3_blockwise(sq):
    """X [4096x7168] 1x128 tiles (0.1% outliers x100), W [7168x7168] 128x128 blocks, bf16 out:
    every code and scale bit for bit; the GEMM on sampled rows."""
    import workloads

    announce("workload3 blockwise full size")
    X, W = workloads.w3_inputs()
    qx, sx = sq.fp8_quantize(X.to(DEV), 0, sq.FP8_SCALE_TILE_1x128)
    qw, sw = sq.fp8_quantize(W.to(DEV), 0, sq.FP8_SCALE_BLOCK_128x128)
    Y = sq.fp8_gemm(qx, 0, sx, sq.FP8_SCALE_TILE_1x128, qw, 0, sw, sq.FP8_SCALE_BLOCK_128x128, sq.OUT_BF16)
    torch.cuda.synchronize()
    announce("workload3 oracle: X tiles, W blocks")
    parts = par_rows(oq.quantize_tile_1x128, f32_np(X), E4)
    oqx = np.concatenate([p[0] for p in parts])
    osx = np.concatenate([p[1] for p in parts], axis=1)
    assert_codes_equal(np_of(qx), oqx, "X tiles")
    assert_f32_bits_equal(np_of(sx), osx, "X tile scale_inv")
    oqw, osw = oq.quantize_block_128x128(f32_np(W), E4)
    assert_codes_equal(np_of(qw), oqw, "W blocks")
    assert_f32_bits_equal(np_of(sw), osw, "W block scale_inv")
    announce("workload3 oracle: GEMM rows")
    rng = np.random.default_rng(3)
    r = _idx(rng, 4096, 48)
    C, S, G = og.gemm_ref(oqx[r], E4, np.ascontiguousarray(osx[:, r]), og.TILE_1x128, oqw, E4, osw, og.BLOCK_128x128)
    check_gemm(_rows(Y, r), C, S, G, 7168, "block", True, "workload3 GEMM")
    em = mm.emulate_gemm(oqx, E4, osx, mm.TILE_1x128, oqw, E4, osw, mm.BLOCK_128x128, rows=r[:2], out_bf16=True)
    assert np.array_equal(_rows(Y, r[:2]).astype(np.float64), em), "workload3 GEMM vs the matrix-core model"


SPIKE4 = 2
STEPS4 = SPIKE4 + H + 2


def test_workload4_fc1_fwd_bwd(sq):
    """X [8192x4096], W [14336x4096], dY [8192x14336]; per-tensor delayed scaling, 20 steps
    (X 4x larger at step 2): every code of q and q^T, the history and the scales each
    step; fwd, dgrad and wgrad GEMMs at the first scaled step and the last."""
    import workloads

    X, W, dY = workloads.w4_inputs()
    Xd, X4d, Wd, dYd = X.to(DEV), (X * 4).to(DEV), W.to(DEV), dY.to(DEV)
    host = {"X": f32_np(X), "X4": f32_np(X) * np.float32(4), "W": f32_np(W), "dY": f32_np(dY)}
    fmts = [E4, E4, E5]
    st = sq.DelayedScalingState(fmts, history_len=H, device=DEV)
    ost = orc.DelayedState(3, H)
    cache = {}

    def oracle_codes(name, scale, fmt):
        key = (name, np.float32(scale).tobytes())
        if key not in cache:
            announce("workload4 oracle codes", name, float(scale))
            q, qT, a = _cast_transpose(host[name], scale, fmt)
            cache[key] = (torch.from_numpy(q).to(DEV), torch.from_numpy(qT).to(DEV), a, q, qT)
        return cache[key]

    rng = np.random.default_rng(4)
    scale0 = []
    for step in range(STEPS4):
        announce("workload4 step", step)
        xname = "X4" if step == SPIKE4 else "X"
        sc = [st.slot(j) for j in range(3)]
        qx, qxT = sq.fp8_cast_transpose(X4d if step == SPIKE4 else Xd, E4, sc[0][0], amax_slot=sc[0][1])
        qw, _ = sq.fp8_quantize(Wd, E4, sq.FP8_SCALE_TENSOR, scale=sc[1][0], amax_slot=sc[1][1])
        _, qwT = sq.fp8_cast_transpose(Wd, E4, sc[1][0])
        qd, qdT = sq.fp8_cast_transpose(dYd, E5, sc[2][0], amax_slot=sc[2][1])
        Y = sq.fp8_gemm(qx, E4, sc[0][2], 0, qw, E4, sc[1][2], 0, sq.OUT_BF16)
        dX = sq.fp8_gemm(qd, E5, sc[2][2], 0, qwT, E4, sc[1][2], 0, sq.OUT_BF16)
        dW = sq.fp8_gemm(qdT, E5, sc[2][2], 0, qxT, E4, sc[0][2], 0, sq.OUT_BF16)
        torch.cuda.synchronize()
        ox = oracle_codes(xname, ost.scale[0], E4)
        ow = oracle_codes("W", ost.scale[1], E4)
        od = oracle_codes("dY", ost.scale[2], E5)
        for got, want, nm in ((qx, ox[0], "X"), (qxT, ox[1], "X^T"), (qw, ow[0], "W"), (qwT, ow[1], "W^T"),
                              (qd, od[0], "dY"), (qdT, od[1], "dY^T")):
            if not torch.equal(got, want):
                assert_codes_equal(np_of(got), np_of(want), f"workload4 {nm} step {step}")
        for j, o in enumerate((ox, ow, od)):
            ost.record(j, o[2])
        assert_f32_bits_equal(np_of(st.amax_history), ost.hist, f"history step {step}")
        if step in (1, STEPS4 - 1):
            si = ost.scale_inv
            r = _idx(rng, 8192, 24)
            r2 = _idx(rng, 14336, 24)
            announce("workload4 oracle: fwd / dgrad / wgrad rows, step", step)
            oqx, oqxT, oqw, oqwT, oqd, oqdT = ox[3], ox[4], ow[3], ow[4], od[3], od[4]
            C, S, G = og.gemm_ref(oqx[r], E4, si[0], 0, oqw, E4, si[1], 0)
            check_gemm(_rows(Y, r), C, S, G, 4096, "tensor", True, f"workload4 fwd step {step}")
            C, S, G = og.gemm_ref(oqd[r], E5, si[2], 0, oqwT, E4, si[1], 0)
            check_gemm(_rows(dX, r), C, S, G, 14336, "tensor", True, f"workload4 dgrad step {step}")
            C, S, G = og.gemm_ref(oqdT[r2], E5, si[2], 0, oqxT, E4, si[0], 0)
            check_gemm(_rows(dW, r2), C, S, G, 8192, "tensor", True, f"workload4 wgrad step {step}")
            _model_rows(Y, oqx, E4, si[0], oqw, E4, si[1], r[:2], "workload4 fwd model")
            _model_rows(dX, oqd, E5, si[2], oqwT, E4, si[1], r[:2], "workload4 dgrad model")
            _model_rows(dW, oqdT, E5, si[2], oqxT, E4, si[0], r2[:2], "workload4 wgrad model")
        st.update()
        ost = orc.delayed_update(ost, fmts)
        torch.cuda.synchronize()
        assert_f32_bits_equal(np_of(st.scale), ost.scale, f"scales after step {step}")
        assert_f32_bits_equal(np_of(st.scale_inv), ost.scale_inv, f"scale_inv after step {step}")
        scale0.append(float(ost.scale[0]))
    spike = scale0[SPIKE4]
    assert all(s == spike for s in scale0[SPIKE4:SPIKE4 + H]), scale0
    assert scale0[SPIKE4 + H] == scale0[SPIKE4 - 1] > spike  # same data before and after: same scale


def test_workload5_mx_and_stream(sq):
    """MX E4M3 8192^3 GEMM (bf16 out) and the 2^28-element amax + cast stream: every code and
    e8m0 byte bit for bit; the GEMM on sampled rows."""
    import workloads

    announce("workload5 MX full size")
    A, B = workloads.w5_inputs()
    qa, ea = sq.fp8_quantize(A.to(DEV), 0, sq.FP8_SCALE_MX_1x32)
    qb, eb = sq.fp8_quantize(B.to(DEV), 0, sq.FP8_SCALE_MX_1x32)
    C = sq.fp8_gemm(qa, 0, ea, sq.FP8_SCALE_MX_1x32, qb, 0, eb, sq.FP8_SCALE_MX_1x32, sq.OUT_BF16)
    torch.cuda.synchronize()
    announce("workload5 oracle: MX A, B")
    pa = par_rows(oq.quantize_mx_1x32, f32_np(A), E4)
    oqa, oea = np.concatenate([p[0] for p in pa]), np.concatenate([p[1] for p in pa])
    assert_codes_equal(np_of(qa), oqa, "A codes")
    assert_codes_equal(np_of(ea).T, oea, "A e8m0")
    pb = par_rows(oq.quantize_mx_1x32, f32_np(B), E4)
    oqb, oeb = np.concatenate([p[0] for p in pb]), np.concatenate([p[1] for p in pb])
    assert_codes_equal(np_of(qb), oqb, "B codes")
    assert_codes_equal(np_of(eb).T, oeb, "B e8m0")
    announce("workload5 oracle: GEMM rows")
    rng = np.random.default_rng(5)
    r = _idx(rng, 8192, 24)
    Cr, S, G = og.gemm_ref(oqa[r], 0, oea[r], og.MX_1x32, oqb, 0, oeb, og.MX_1x32)
    check_gemm(_rows(C, r), Cr, S, G, 8192, "mx", True, "workload5 MX GEMM")
    em = mm.emulate_gemm(oqa, E4, oea, mm.MX_1x32, oqb, E4, oeb, mm.MX_1x32, rows=r[:2], out_bf16=True)
    frac = float(np.mean(_rows(C, r[:2]).astype(np.float64) == em))
    print(f"[model] workload5 MX rows: {frac:.5f} bit-exact", flush=True)
    assert frac >= 0.99, f"workload5 MX GEMM: {frac:.4f} of outputs equal the matrix-core model"
    del A, B, qa, qb, C
    announce("workload5 stream 2^28 amax + cast")
    T = workloads.w5_stream()
    s = np.float32(448.0) / np.float32(5.5)
    slot = torch.zeros(1, device=DEV)
    q, _ = sq.fp8_quantize(T.to(DEV), 0, sq.FP8_SCALE_TENSOR, scale=_scal(s), amax_slot=slot)
    torch.cuda.synchronize()
    t = f32_np(T).reshape(1 << 14, 1 << 14)
    parts = par_rows(oq.quantize_tensor, t, s, E4, chunks=64)
    want = np.concatenate([p[0] for p in parts]).reshape(-1)
    assert_f32_bits_equal(np_of(slot), [np.max(np.array([p[1] for p in parts], np.float32))], "stream amax")
    assert_codes_equal(np_of(q), want, "stream codes (all 2^28)")
