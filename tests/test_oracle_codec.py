"""Pins of the oracle's FP8 / bf16 / e8m0 codec (CPU only).

Pinned against: the format facts the pages print (tests/golden/format_facts.txt),
brute force over all 256 codes against an independent scalar decoder, the
exhaustive bf16 -> FP8 mapping against an independent exact-rational scalar
encoder, and PyTorch's own float8 / bfloat16 conversions (a library routine)
wherever those are defined the same way (in-range values).
"""

import math

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import fp8

E4M3, E5M2 = fp8.E4M3, fp8.E5M2
FMTS = {"E4M3": E4M3, "E5M2": E5M2}


def test_format_facts_from_pages():
    for fact, fmt, value, expected in read_golden("format_facts.txt"):
        if fact == "fmax":
            f = FMTS[fmt]
            assert fp8.FMAX[f] == float(expected)
            codes, vals = fp8.positive_grid(f)
            assert vals[-1] == float(expected)
        elif fact in ("ebits", "mbits"):
            f = FMTS[fmt]
            # count distinct exponent / mantissa fields by decoding: 2^mbits codes per binade
            codes, vals = fp8.positive_grid(f)
            normal = vals[vals >= 1.0]
            per_binade = np.sum((normal >= 1.0) & (normal < 2.0))
            mb = int(round(math.log2(per_binade)))
            if fact == "mbits":
                assert mb == int(expected)
            else:
                assert 7 - mb == int(expected)
        elif fact == "round":
            assert fp8.to_bf16(np.float32(float(value))) == np.float32(float(expected))
        elif fact == "spacing":
            v = np.float32(float(value))
            lo = fp8.to_bf16(v)
            up = fp8.bf16_bits_to_f32(fp8.bf16_round_bits(v) + np.uint16(1))
            assert float(np.asarray(up - lo).reshape(-1)[0]) == float(expected)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_all_codes_vs_scalar(fmt):
    codes = np.arange(256, dtype=np.uint8)
    vec = fp8.decode(codes, fmt)
    for c in range(256):
        s = fp8.decode_scalar(c, fmt)
        if math.isnan(s):
            assert math.isnan(vec[c])
        else:
            assert vec[c] == s, c


def test_code_counts_and_anchors():
    v4 = fp8.decode(np.arange(128, dtype=np.uint8), E4M3)
    v5 = fp8.decode(np.arange(128, dtype=np.uint8), E5M2)
    assert np.sum(np.isfinite(v4) & (v4 > 0)) == 126
    assert np.sum(np.isfinite(v5) & (v5 > 0)) == 123
    assert v4[0x38] == 1.0 and v5[0x3C] == 1.0
    assert v4[0x44] == 3.0 and v4[0x76] == 224.0 and v4[0x7E] == 448.0
    assert v5[0x7B] == 57344.0 and np.isinf(v5[0x7C]) and np.isnan(v4[0x7F])
    assert v4[0x01] == 2.0 ** -9 and v5[0x01] == 2.0 ** -16


@pytest.mark.parametrize("fmt,tdtype", [(E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)])
def test_decode_matches_torch(fmt, tdtype):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(tdtype).to(torch.float64).numpy()
    o = fp8.decode(codes.numpy(), fmt)
    assert np.array_equal(np.isnan(t), np.isnan(o))
    ok = ~np.isnan(o)
    assert np.array_equal(t[ok], o[ok])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_roundtrip_every_finite_code(fmt):
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.decode(codes, fmt)
    finite = np.isfinite(vals)
    back = fp8.encode(vals[finite].astype(np.float32), fmt)
    assert np.array_equal(back, codes[finite])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_midpoints_go_to_even_code(fmt):
    codes, vals = fp8.positive_grid(fmt)
    for i in range(len(vals) - 1):
        mid = np.float32((vals[i] + vals[i + 1]) / 2)
        assert float(mid) == (vals[i] + vals[i + 1]) / 2  # exact in float32
        even = codes[i] if codes[i] % 2 == 0 else codes[i + 1]
        for sign in (1, -1):
            c = fp8.encode(np.float32(sign * mid), fmt)
            assert c == (even | (0x80 if sign < 0 else 0))
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert fp8.encode(below, fmt) == codes[i]
        assert fp8.encode(above, fmt) == codes[i + 1]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_exhaustive_bf16_vs_scalar(fmt):
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    vec = fp8.encode(x, fmt)
    scal = np.array([fp8.encode_scalar(float(v), fmt) for v in x], dtype=np.uint8)
    assert np.array_equal(vec, scal)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_random_scaled_vs_scalar(fmt):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(4000) * rng.choice([1e-3, 1.0, 100.0, 3e4], 4000)).astype(np.float32)
    s = np.float32(1.8666666746139526)
    v = (x * s).astype(np.float32)
    vec = fp8.encode(v, fmt)
    scal = np.array([fp8.encode_scalar(float(t), fmt) for t in v], dtype=np.uint8)
    assert np.array_equal(vec, scal)


@pytest.mark.parametrize("fmt,tdtype", [(E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)])
def test_encode_matches_torch_in_range(fmt, tdtype):
    # torch rounds to nearest even; it does not saturate, so compare where |v| <= fmax
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= fp8.FMAX[fmt])]
    bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    bf = bf[np.isfinite(bf) & (np.abs(bf) <= fp8.FMAX[fmt])]
    for arr in (x, bf):
        t = torch.from_numpy(arr.copy()).to(tdtype).view(torch.uint8).numpy()
        assert np.array_equal(fp8.encode(arr, fmt), t)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_saturation_and_special_value_readings(fmt):
    top = 0x7E if fmt == E4M3 else 0x7B
    f = np.float32
    assert fp8.encode(f(fp8.FMAX[fmt] * 1.01), fmt) == top  # "clips at 448"
    assert fp8.encode(f(1e30), fmt) == top
    assert fp8.encode(f(-1e30), fmt) == top | 0x80
    assert fp8.encode(f(np.inf), fmt) == top
    assert fp8.encode(f(-np.inf), fmt) == top | 0x80
    assert fp8.encode(f(np.nan), fmt) == 0x7F
    assert fp8.encode(-f(np.nan), fmt) == 0xFF
    assert fp8.encode(f(0.0), fmt) == 0x00
    assert fp8.encode(f(-0.0), fmt) == 0x80
    assert fp8.encode(f(-1e-30), fmt) == 0x80


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x3F808000, 0x3F818000, 0x7F7F8000, 0x7F7FFFFF, 0xFF7F8000, 0x00008000,
                         0x00018000, 0x7F800000, 0x80000000, 0x43808000], dtype=np.uint32)
    x = np.concatenate([u, specials]).view(np.float32)
    ours = fp8.bf16_round_bits(x)
    t = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], t[~nan])
    assert np.all(np.isnan(fp8.bf16_bits_to_f32(ours[nan])))


def test_e8m0_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    o = fp8.e8m0_decode(codes.numpy())
    assert np.array_equal(np.isnan(t), np.isnan(o))
    assert np.array_equal(t[~np.isnan(t)], o[~np.isnan(o)])
