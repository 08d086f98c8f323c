"""Property tests of the oracle over arbitrary inputs (CPU only, hypothesis).

Each property is checked against something other than the oracle's own formula:
- the vectorised encoder against the exact-rational scalar encoder, for any float32 (the
  exhaustive pins cover bf16 inputs; these cover the fp32 products the casts round);
- nearest-value rounding against a brute-force search of the finite grid, in exact rationals,
  and saturation beyond the format's maximum ([L] Worked example, step 02: clipping at 448);
- monotonicity of encode-then-decode;
- the MX rule against its definition (the smallest integer E with amax <= fmax * 2^E);
- the blockwise current scale against the invariant that the block maximum lands on the
  format's largest code;
- the delayed recipe's scale against a sliding window of the last H amaxes kept in a deque
  ([T] recipe cell: amax_history_len, "max"), i.e. an independent statement of the ring;
- bf16 round-to-nearest-even against PyTorch's float -> bfloat16 conversion.
"""

import math
from collections import deque
from fractions import Fraction

import numpy as np
import torch
from hypothesis import given, settings, strategies as st

from oracle import fp8, recipe

def _f32(x: float) -> float:
    return float(np.float32(x))


F32 = st.floats(width=32, allow_nan=False, allow_infinity=False)
FMTS = st.sampled_from([fp8.E4M3, fp8.E5M2])
SETTINGS = settings(max_examples=300, deadline=None)
TOP = {fp8.E4M3: 0x7E, fp8.E5M2: 0x7B}


@SETTINGS
@given(v=F32, fmt=FMTS)
def test_encode_agrees_with_exact_rational_encoder(v, fmt):
    assert int(fp8.encode(np.float32(v), fmt)) == fp8.encode_scalar(v, fmt)


@SETTINGS
@given(v=F32, fmt=FMTS)
def test_encode_picks_a_nearest_grid_value_and_saturates(v, fmt):
    c = int(fp8.encode(np.float32(v), fmt))
    assert (c >> 7) == (1 if math.copysign(1.0, v) < 0 else 0), "sign bit (zero keeps its sign)"
    mag = abs(fp8.decode_scalar(c & 0x7F, fmt))
    fmax = fp8.FMAX[fmt]
    if abs(v) >= fmax:
        assert mag == fmax
        return
    _, grid = fp8.positive_grid(fmt)
    a = abs(Fraction(v))
    best = min(abs(a - Fraction(float(g))) for g in grid)
    assert abs(a - Fraction(mag)) == best


@SETTINGS
@given(a=F32, b=F32, fmt=FMTS)
def test_encode_then_decode_is_monotone(a, b, fmt):
    lo, hi = (a, b) if a <= b else (b, a)
    dlo = fp8.decode(fp8.encode(np.float32(lo), fmt), fmt)
    dhi = fp8.decode(fp8.encode(np.float32(hi), fmt), fmt)
    assert dlo <= dhi


@SETTINGS
@given(g=st.floats(min_value=_f32(1e-40), max_value=_f32(3.0e38), width=32), fmt=FMTS)
def test_mx_exponent_is_the_smallest_fitting_power_of_two(g, fmt):
    E = int(recipe.mx_exponent(np.float32(g), fmt)) - 127
    fmax = fp8.FMAX[fmt]
    g = float(np.float32(g))
    if -127 < E < 127:  # not clamped: the defining inequality, in exact double arithmetic
        assert g <= math.ldexp(fmax, E)
        assert g > math.ldexp(fmax, E - 1)
    elif E == -127:
        assert g <= math.ldexp(fmax, -127)


@SETTINGS
@given(a=st.floats(min_value=_f32(1e-30), max_value=_f32(3.0e38), width=32), fmt=FMTS)
def test_current_scale_puts_the_block_maximum_on_the_top_code(a, fmt):
    a = np.float32(a)
    s, s_inv = recipe.current_scale(a, fmt)
    code = int(fp8.encode(np.float32(a * np.float32(s)), fmt))
    assert code == TOP[fmt]
    assert np.float32(s_inv) == np.float32(np.float32(1.0) / np.float32(s))


@SETTINGS
@given(H=st.integers(1, 24), fmt=FMTS,
       seq=st.lists(st.one_of(st.just(0.0), st.floats(min_value=_f32(1e-20), max_value=_f32(1e20), width=32)),
                    min_size=1, max_size=48))
def test_delayed_scale_follows_the_last_H_amaxes(H, fmt, seq):
    state = recipe.DelayedState(1, H)
    window = deque(maxlen=H)
    fmax = np.float32(fp8.FMAX[fmt])
    scale = np.float32(1.0)
    for a in seq:
        a = np.float32(a)
        state.record(0, a)
        window.append(a)
        state = recipe.delayed_update(state, [fmt])
        m = max(window)
        if m > 0:
            q = float(fmax) / float(m)  # exact quotient, rounded once to float32 below
            scale = np.float32(q) if q <= float(np.finfo(np.float32).max) else np.finfo(np.float32).max
        assert state.scale[0] == scale
        assert state.scale_inv[0] == np.float32(np.float32(1.0) / scale)


@SETTINGS
@given(v=F32)
def test_bf16_rounding_matches_pytorch(v):
    ours = int(np.asarray(fp8.bf16_round_bits(np.float32(v))).reshape(-1)[0])
    t = torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
    assert ours == t
