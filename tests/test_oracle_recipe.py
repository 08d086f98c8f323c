"""Pins of the oracle's amax / scale / delayed-recipe / current-scaling / MX rules (CPU only)."""

import numpy as np
import pytest

from conftest import read_golden
from oracle import fp8, quantize, recipe

E4M3, E5M2 = fp8.E4M3, fp8.E5M2
f32 = np.float32


def test_worked_example_scale_from_pages():
    """Lesson worked example: scale ~ 448/240; 120 -> ~224; 300 -> ~560, clips at 448."""
    for amax, fmax, value, scaled, result in read_golden("worked_example_scale.txt"):
        s, s_inv = recipe.current_scale(f32(float(amax)), E4M3)
        assert float(fmax) == fp8.FMAX[E4M3]
        assert abs(float(s) - 1.87) < 0.005  # "scale ~ 1.87"
        v = f32(f32(float(value)) * s)
        assert abs(float(v) - float(scaled)) < 0.01 * float(scaled)
        q, _ = quantize.quantize_tensor(np.array([float(value)], np.float32), s, E4M3)
        assert fp8.decode(q, E4M3)[0] == float(result)
    # the exact codes: 120 * fp32(448/240) rounds to 224.0 -> 0x76; 300 saturates -> 0x7E
    s = f32(448.0) / f32(240.0)
    q, a = quantize.quantize_tensor(np.array([120.0, 300.0, -300.0], np.float32), s, E4M3)
    assert list(q) == [0x76, 0x7E, 0xFE] and a == 300.0


def _run_delayed(amaxes, H, fmt=E4M3, margin=0):
    """Scales used at each step when tensor t has amax amaxes[t]."""
    st = recipe.DelayedState(1, H)
    used = []
    for a in amaxes:
        used.append(float(st.scale[0]))
        st.record(0, a)
        st = recipe.delayed_update(st, [fmt], margin)
    return used, st


def test_delayed_initial_state_and_lag():
    st = recipe.DelayedState(3, 16)
    assert st.hist.shape == (16, 3)
    assert np.all(st.hist == 0) and np.all(st.scale == 1) and np.all(st.scale_inv == 1)
    # a tensor never scales itself: step 0 uses the initial scale 1
    used, _ = _run_delayed([240.0, 240.0], 16)
    assert used[0] == 1.0 and used[1] == float(f32(448) / f32(240))


def test_delayed_window_closed_form():
    """scale_{t+1} = fmax / max(amax_{t-H+1..t}) -- the ring's closed form."""
    rng = np.random.default_rng(0)
    for H in (1, 4, 16):
        amaxes = rng.uniform(0.5, 8.0, 60).astype(np.float32)
        used, _ = _run_delayed(amaxes, H)
        for t in range(1, 60):
            m = amaxes[max(0, t - H):t].max()
            assert used[t] == float(f32(448.0) / f32(m)), (H, t)


def test_delayed_spike_clips_then_ages_out():
    """Lesson worked example 02 + delayed lag: the spike step clips; its amax rules for exactly H steps."""
    H = 16
    amaxes = [240.0] * 20 + [300.0] + [240.0] * 20
    used, _ = _run_delayed(amaxes, H)
    s_old = float(f32(448) / f32(240))
    s_new = float(f32(448) / f32(300))
    assert used[20] == s_old  # the spike is quantised with the stale scale
    q, _ = quantize.quantize_tensor(np.array([300.0], np.float32), used[20], E4M3)
    assert q[0] == 0x7E  # clips at 448
    assert all(u == s_new for u in used[21:21 + H])
    assert used[21 + H] == s_old
    # at the new scale 120 maps to 179.2, which rounds to 176 (0x73)
    q, _ = quantize.quantize_tensor(np.array([120.0], np.float32), s_new, E4M3)
    assert q[0] == 0x73


def test_delayed_margin_is_power_of_two():
    for k in range(0, 5):
        used, st = _run_delayed([3.0, 3.0], 16, margin=k)
        base = f32(448) / f32(3)
        assert used[1] == float(base) * 2.0 ** -k
        assert st.scale_inv[0] == f32(1) / f32(used[1])


def test_delayed_e5m2_slots_and_many_slots():
    st = recipe.DelayedState(3, 4)
    for j, a in enumerate([2.0, 4.0, 1e-3]):
        st.record(j, a)
    st = recipe.delayed_update(st, [E4M3, E4M3, E5M2])
    assert st.scale[0] == f32(448) / f32(2)
    assert st.scale[1] == f32(448) / f32(4)
    assert st.scale[2] == f32(57344) / f32(1e-3)
    assert np.all(st.hist[0] == 0) and np.all(st.hist[-1] == np.array([2.0, 4.0, 1e-3], np.float32))


@pytest.mark.parametrize("bad", [0.0, np.inf, np.nan])
def test_delayed_nonfinite_or_zero_window_keeps_scale(bad):
    used, st = _run_delayed([2.0], 2)
    s = st.scale[0]
    st2 = st.copy()
    st2.record(0, bad)
    st2.hist[1:, :] = 0 if bad == 0.0 else st2.hist[1:, :]
    st3 = recipe.delayed_update(st2, [E4M3])
    if bad == 0.0:
        assert st3.scale[0] == s  # window max 0 -> unchanged
    else:
        assert st3.scale[0] == s and st3.scale_inv[0] == st.scale_inv[0]


def test_record_is_max_and_nan_propagates():
    st = recipe.DelayedState(1, 4)
    st.record(0, 3.0)
    st.record(0, 2.0)
    assert st.hist[0, 0] == 3.0
    st.record(0, np.nan)
    assert np.isnan(st.hist[0, 0])


def test_amax_definition():
    x = np.array([0.0, -0.0, -5.5, 2.0], np.float32)
    assert recipe.amax(x) == 5.5
    assert np.isnan(recipe.amax(np.array([1.0, np.nan], np.float32)))
    assert recipe.amax(np.array([-np.inf, 1.0], np.float32)) == np.inf
    assert recipe.amax(np.zeros(0, np.float32)) == 0.0


def test_scale_overflow_clamps_to_flt_max():
    s, s_inv = recipe.current_scale(f32(1e-40), E4M3)
    assert s == recipe.FLT_MAX and np.isfinite(s_inv)
    used, st = _run_delayed([1e-40, 1e-40], 4)
    assert st.scale[0] == recipe.FLT_MAX


def test_current_scaling_block_max_hits_fmax():
    """Every non-zero tile has an element of magnitude exactly fmax (its amax element)."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 512)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    q, sinv = quantize.quantize_tile_1x128(x, E4M3)
    t = q.reshape(64, 4, 128) & 0x7F
    assert np.all(t.max(axis=2) == 0x7E)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    qw, sw = quantize.quantize_block_128x128(w, E4M3)
    b = (qw & 0x7F).reshape(2, 128, 3, 128)
    assert np.all(b.max(axis=(1, 3)) == 0x7E)
    assert sinv.shape == (4, 64) and sw.shape == (2, 3)


def test_outlier_spoils_only_its_own_tile():
    """Course page: with per-block scales an outlier spoils only its own block."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    y = x.copy()
    y[3, 200] *= 100.0
    qx, sx = quantize.quantize_tile_1x128(x, E4M3)
    qy, sy = quantize.quantize_tile_1x128(y, E4M3)
    diff = qx != qy
    assert diff[3, 128:256].any()
    diff[3, 128:256] = False
    assert not diff.any()
    # per-tensor scaling of the same data: the outlier changes codes everywhere
    st = recipe.current_scale(recipe.amax(x), E4M3)[0]
    sty = recipe.current_scale(recipe.amax(y), E4M3)[0]
    ax, _ = quantize.quantize_tensor(x, st, E4M3)
    ay, _ = quantize.quantize_tensor(y, sty, E4M3)
    assert (ax != ay).mean() > 0.5


def test_zero_tile_gets_unit_scale():
    x = np.zeros((2, 256), np.float32)
    x[1, 130] = 2.0
    q, s = quantize.quantize_tile_1x128(x, E4M3)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert s[1, 1] == f32(1) / (f32(448) / f32(2))
    assert np.all(q[0] == 0)


def test_mx_exponent_closed_form_boundaries():
    """E = e - 8 when amax <= 1.75 * 2^e, else e - 7 (E4M3); 15 in place of 8 for E5M2."""
    for fmt, off in ((E4M3, 8), (E5M2, 15)):
        for e in range(-100, 100, 7):
            g = f32(1.75 * 2.0 ** e)
            assert int(recipe.mx_exponent(g, fmt)) - 127 == max(-127, e - off)
            g_up = np.nextafter(g, f32(np.inf))
            assert int(recipe.mx_exponent(g_up, fmt)) - 127 == max(-127, e - off + 1)
            g_pow = f32(2.0 ** e)
            assert int(recipe.mx_exponent(g_pow, fmt)) - 127 == max(-127, e - off)


def test_mx_group_max_decodes_into_upper_half_of_range():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((32, 256)) * np.exp2(rng.integers(-40, 40, (32, 1)))).astype(np.float32)
    q, codes = quantize.quantize_mx_1x32(x, E4M3)
    d = fp8.decode(q, E4M3).reshape(32, 8, 32)
    gm = np.abs(d).max(axis=2)
    # before rounding the scaled group max lies in (fmax/2, fmax]; the FP8 code can round down onto fmax/2
    g = np.abs(x.reshape(32, 8, 32)).max(axis=2).astype(np.float64)
    scaled = g * np.exp2(-(codes.astype(np.float64) - 127))
    assert np.all(scaled > 224.0) and np.all(scaled <= 448.0)
    assert np.all(gm >= 224.0) and np.all(gm <= 448.0)
    # nothing saturates: dequantised value equals the float32 product's rounding
    scale = fp8.e8m0_decode(codes)
    back = (d * scale[:, :, None]).reshape(32, 256)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 + 1e-300)


def test_mx_zero_and_nan_groups():
    x = np.zeros((1, 64), np.float32)
    x[0, 40] = np.nan
    q, codes = quantize.quantize_mx_1x32(x, E4M3)
    assert codes[0, 0] == 0 and codes[0, 1] == 255
    assert q[0, 40] == 0x7F and np.all(q[0, :32] == 0)


# --------------------------------------------------------------------------- blockwise transposes


def _bw_data(seed, rows=256, cols=384):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-8, 8, (1, cols))).astype(np.float32)  # column-dependent magnitudes
    return x


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_column_runs_max_hits_fmax(fmt):
    """Every non-zero 128x1 run of the transposed copy holds a code of magnitude fmax (its
    amax element), and its scale is fmax / that run's amax."""
    x = _bw_data(21)
    x[128:256, 5] = 0.0  # a zero run: unit scale
    _, _, qT, sT = quantize.cast_transpose_blockwise(x, fmt, 1)
    fmax_code = 0x7E if fmt == E4M3 else 0x7B
    for c in range(x.shape[1]):
        for rb in range(2):
            run = qT[c, rb * 128:(rb + 1) * 128]
            a = np.abs(x[rb * 128:(rb + 1) * 128, c]).max()
            if a == 0:
                assert sT[rb, c] == 1.0 and np.all((run & 0x7F) == 0)
            else:
                assert np.any((run & 0x7F) == fmax_code)
                assert sT[rb, c] == f32(1) / (f32(fp8.FMAX[fmt]) / f32(a))


def test_column_runs_outlier_spoils_only_its_run():
    """An outlier changes the codes of its own 128x1 run in the transposed copy and of its own
    1x128 run in the forward copy, and nothing else."""
    x = _bw_data(22)
    y = x.copy()
    y[200, 7] *= 1000.0
    q0, _, t0, _ = quantize.cast_transpose_blockwise(x, E4M3, 1)
    q1, _, t1, _ = quantize.cast_transpose_blockwise(y, E4M3, 1)
    dq = np.argwhere(q0 != q1)
    assert len(dq) and np.all(dq[:, 0] == 200) and np.all(dq[:, 1] // 128 == 0)
    dt = np.argwhere(t0 != t1)
    assert len(dt) and np.all(dt[:, 0] == 7) and np.all(dt[:, 1] // 128 == 1)


def test_column_runs_brute_force():
    x = _bw_data(23, rows=128, cols=128)
    _, _, qT, sT = quantize.cast_transpose_blockwise(x, E4M3, 1)
    for c in range(0, 128, 13):
        a = np.abs(x[:, c]).max()
        s = f32(448.0) / f32(a)
        for r in range(0, 128, 11):
            assert qT[c, r] == fp8.encode_scalar(float(f32(x[r, c] * s)), E4M3)


def test_block_transpose_is_transpose_of_codes_and_scales():
    x = _bw_data(24)
    q, s, qT, sT = quantize.cast_transpose_blockwise(x, E4M3, 2)
    q2, s2 = quantize.quantize_block_128x128(x.T, E4M3)  # the same blocks, seen transposed
    assert np.array_equal(qT, q.T) and np.array_equal(sT, s.T)
    assert np.array_equal(qT, q2) and np.array_equal(sT, s2)


# --------------------------------------------------------------------------- cast diagnostics


def test_diagnostics_worked_example_spike_is_one_saturation():
    """Worked example: with the scale 448/240, 120 fits and 300 clips at 448 -> one saturation."""
    rows = [[float(v) for v in r] for r in read_golden("worked_example_scale.txt")]
    amax, fmax = rows[0][0], rows[0][1]
    s = f32(fmax) / f32(amax)
    x = np.array([r[2] for r in rows], np.float32)
    q, _ = quantize.quantize_tensor(x, s, E4M3)
    assert quantize.cast_diagnostics(x, s, E4M3) == (1, 0, 0)
    assert fp8.decode(q, E4M3)[1] == 448.0


@pytest.mark.parametrize("fmt,tiny", [(E4M3, -9), (E5M2, -16)])
def test_diagnostics_underflow_boundary(fmt, tiny):
    """Half the smallest subnormal ties to the even code 0 (underflow); just above it rounds
    up to the smallest subnormal; zeros of either sign are not underflows."""
    half = np.exp2(f32(tiny - 1))
    x = np.array([half, half * f32(1 + 2 ** -20), -half / 2, 0.0, -0.0, np.exp2(f32(tiny))], np.float32)
    assert quantize.cast_diagnostics(x, f32(1), fmt) == (0, 2, 0)


def test_diagnostics_specials_and_code_consistency():
    rng = np.random.default_rng(31)
    x = (rng.standard_normal(4096) * 100).astype(np.float32)
    x[:3] = [np.inf, -np.inf, np.nan]
    s = f32(2.0)
    sat, und, nan = quantize.cast_diagnostics(x, s, E4M3)
    q, _ = quantize.quantize_tensor(x, s, E4M3)
    with np.errstate(over="ignore", invalid="ignore"):
        y = x * s
    clipped = np.isfinite(x) & (np.abs(y) > 448)
    assert nan == 1 and sat == int(clipped.sum()) + 2 and und == 0
    assert np.all((q[clipped] & 0x7F) == 0x7E)
