"""Pins of the oracle's number formats (CPU only).

Each test checks the oracle against something other than itself: the OCP format
landmarks in tests/golden, exhaustive enumeration of all 256 FP8 codes,
hardware/library conversions (numpy binary32/binary16, torch bfloat16 and torch
FP8 casts inside the finite range) and closed-form brackets of the E8M0 rule.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_value(s):
    return {"nan": math.nan, "inf": math.inf, "-inf": -math.inf}.get(s, None) if s in (
        "nan", "inf", "-inf") else float(s)


def test_fp8_landmarks_decode_and_encode():
    n = 0
    with open(os.path.join(GOLDEN, "fp8_landmarks.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, code, val = line.split()
            fmt = F.FORMATS[name]
            code = int(code, 16)
            val = _parse_value(val)
            got = float(F.fp8_decode(np.array([code]), fmt)[0])
            if math.isnan(val):
                assert math.isnan(got), (name, hex(code))
                continue
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (name, hex(code), got)
            if math.isfinite(val):
                assert int(F.fp8_quantize(np.array([val]), fmt)[0]) == code, (name, hex(code))
            n += 1
    assert n >= 20


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2], ids=["e4m3", "e5m2"])
def test_fp8_exhaustive_roundtrip(fmt):
    codes = np.arange(256)
    vals = F.fp8_decode(codes, fmt)
    finite = np.isfinite(vals)
    re = F.fp8_quantize(vals[finite], fmt)
    assert np.array_equal(re.astype(np.int64), codes[finite])
    # number of finite codes fixed by the format definitions
    assert int(finite.sum()) == (254 if fmt is F.E4M3 else 248)


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2], ids=["e4m3", "e5m2"])
def test_fp8_positive_codes_monotone_and_max(fmt):
    vals = F.fp8_decode(np.arange(128), fmt)
    fin = vals[np.isfinite(vals)]
    assert np.all(np.diff(fin) > 0)
    assert fin[-1] == fmt.max_finite


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2], ids=["e4m3", "e5m2"])
def test_fp8_midpoints_round_to_even_code(fmt):
    vals = F.fp8_decode(np.arange(128), fmt)
    fin = np.isfinite(vals)
    codes = np.arange(128)[fin]
    v = vals[fin]
    for i in range(len(v) - 1):
        mid = 0.5 * (v[i] + v[i + 1])
        even = codes[i] if codes[i] % 2 == 0 else codes[i + 1]
        assert int(F.fp8_quantize(np.array([mid]), fmt)[0]) == even
        assert int(F.fp8_quantize(np.array([-mid]), fmt)[0]) == even | 0x80
        # just off the midpoint: the nearer neighbour
        eps = (v[i + 1] - v[i]) * 1e-6
        assert int(F.fp8_quantize(np.array([mid - eps]), fmt)[0]) == codes[i]
        assert int(F.fp8_quantize(np.array([mid + eps]), fmt)[0]) == codes[i + 1]


def test_fp8_saturation():
    e4, e5 = F.E4M3, F.E5M2
    for v, c in [(448.0, 0x7E), (464.0, 0x7E), (470.0, 0x7E), (480.0, 0x7E), (1e6, 0x7E),
                 (-500.0, 0xFE), (np.inf, 0x7E)]:
        assert int(F.fp8_quantize(np.array([v]), e4)[0]) == c, v
    for v, c in [(57344.0, 0x7B), (61440.0, 0x7B), (1e9, 0x7B), (-7e4, 0xFB)]:
        assert int(F.fp8_quantize(np.array([v]), e5)[0]) == c, v


def test_fp8_subnormals_and_zero():
    e4 = F.E4M3
    tiny = 2.0 ** -9
    assert int(F.fp8_quantize(np.array([tiny * 0.5]), e4)[0]) == 0x00      # tie -> even (0)
    assert int(F.fp8_quantize(np.array([tiny * 0.5000001]), e4)[0]) == 0x01
    assert int(F.fp8_quantize(np.array([tiny * 1.5]), e4)[0]) == 0x02      # tie 1.5 -> 2
    assert int(F.fp8_quantize(np.array([-1e-30]), e4)[0]) == 0x80          # sign kept
    assert int(F.fp8_quantize(np.array([0.0]), e4)[0]) == 0x00


@pytest.mark.parametrize("name,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_matches_torch_cast_inside_range(name, tdt):
    """torch's FP8 cast rounds nearest-even but does not saturate, so compare only
    on values already clamped to the finite range."""
    fmt = F.FORMATS[name]
    g = torch.Generator().manual_seed(11)
    v = torch.cat([torch.randn(200000, generator=g) * s for s in (0.01, 1.0, 30.0, 3000.0)])
    v = v.clamp(-fmt.max_finite, fmt.max_finite).to(torch.float32)
    ref = v.to(tdt).view(torch.uint8).numpy()
    ours = F.fp8_quantize(v.numpy().astype(np.float64), fmt)
    assert np.array_equal(ref, ours)


def test_bf16_rounding_matches_torch_and_ties():
    g = torch.Generator().manual_seed(5)
    v = torch.randn(300000, generator=g, dtype=torch.float32) * 37.0
    ref = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = F.encode_storage(v.numpy().astype(np.float64), "bf16")
    assert np.array_equal(ref, ours)
    # exact ties: binary32 patterns whose low 16 bits are 0x8000
    hi = np.arange(0x3F80, 0x3FA0, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32).astype(np.float64)
    got = F.encode_storage(ties, "bf16")
    expect = np.where(hi % 2 == 0, hi, hi + 1).astype(np.uint16)
    assert np.array_equal(got, expect)


def test_f32_and_f16_rounding_match_numpy():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))
    assert np.array_equal(F.to_f32(v), v.astype(np.float32).astype(np.float64))
    w = (rng.standard_normal(200000) * 300).astype(np.float32)
    assert np.array_equal(F.encode_storage(w.astype(np.float64), "f16"), w.astype(np.float16))


def test_decode_storage_bf16_matches_torch():
    g = torch.Generator().manual_seed(9)
    t = torch.randn(1000, generator=g).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.decode_storage(bits, "bf16"), t.to(torch.float64).numpy())


def test_e8m0_golden_examples():
    n = 0
    with open(os.path.join(GOLDEN, "mx_e8m0_examples.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "code":
                _, name, amax, elem, code = parts
                x = int(F.e8m0_exponent(np.array([float(amax)]), name)[0])
                scaled = float(elem) * 2.0 ** (-x)
                assert int(F.fp8_quantize(np.array([scaled]), F.FORMATS[name])[0]) == int(code, 16)
            else:
                name, amax, byte = parts
                assert int(F.e8m0_exponent(np.array([float(amax)]), name)[0]) + 127 == int(byte), line
            n += 1
    assert n >= 15


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_e8m0_floor_rule_at_powers_of_two(name):
    emax = F.MX_EMAX[name]
    for k in range(-120, 120):
        p = 2.0 ** k
        below = math.nextafter(p, 0.0)
        above = math.nextafter(p, math.inf)
        x = F.e8m0_exponent(np.array([p, below, above]), name)
        expect = [k - emax, k - 1 - emax, k - emax]
        assert list(x) == [min(127, max(-127, e)) for e in expect]


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_e8m0_bracket_and_clamp(name):
    emax = F.MX_EMAX[name]
    rng = np.random.default_rng(1)
    a = np.exp(rng.uniform(-60, 60, 100000))   # inside the unclamped range
    x = F.e8m0_exponent(a, name)
    # closed form: 2^(X+emax) <= a < 2^(X+emax+1)
    assert np.all(np.ldexp(1.0, x + emax) <= a) and np.all(a < np.ldexp(1.0, x + emax + 1))
    # clamp at both ends of the E8M0 range
    assert int(F.e8m0_exponent(np.array([1e-300]), name)[0]) == -127
    assert int(F.e8m0_exponent(np.array([0.0]), name)[0]) == -127
    assert int(F.e8m0_exponent(np.array([1e300]), name)[0]) == 127


def test_mx_scaled_block_max_lies_in_top_binade():
    """Under the floor rule the block maximum scales into [2^emax, 2^(emax+1)), so it
    either lands on a top-binade code or saturates to the largest finite code."""
    rng = np.random.default_rng(2)
    a = np.exp(rng.uniform(-30, 30, 10000))
    for name in ("e4m3", "e5m2"):
        x = F.e8m0_exponent(a, name)
        s = a * np.ldexp(1.0, -x)
        emax = F.MX_EMAX[name]
        assert np.all(s >= 2.0 ** emax) and np.all(s < 2.0 ** (emax + 1))


def test_e8m0_ceil_golden_examples():
    n = 0
    with open(os.path.join(GOLDEN, "mx_e8m0_ceil_examples.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "code":
                _, name, amax, elem, code = parts
                x = int(F.e8m0_exponent(np.array([float(amax)]), name, "ceil")[0])
                scaled = float(elem) * 2.0 ** (-x)
                assert int(F.fp8_quantize(np.array([scaled]), F.FORMATS[name])[0]) == int(code, 16), line
            else:
                name, amax, byte = parts
                assert int(F.e8m0_exponent(np.array([float(amax)]), name, "ceil")[0]) + 127 == int(byte), line
            n += 1
    assert n >= 15


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_e8m0_ceil_is_the_smallest_exponent_that_does_not_saturate(name):
    """Brute force: X is the smallest integer with a * 2^-X <= max, checked by trying X and
    X - 1 in exact power-of-two arithmetic, on random maxima and on the boundaries
    1.75 * 2^k (where the significand equals that of the largest finite value) and their
    float64 neighbours."""
    fmax = F.FORMATS[name].max_finite
    rng = np.random.default_rng(3)
    k = np.arange(-100, 100)
    edge = np.ldexp(1.75, k)
    a = np.concatenate([np.exp(rng.uniform(-60, 60, 50000)), edge, np.nextafter(edge, 0.0),
                        np.nextafter(edge, np.inf), np.ldexp(1.0, k), np.nextafter(np.ldexp(1.0, k), 0.0)])
    x = F.e8m0_exponent(a, name, "ceil")
    assert np.all(a * np.ldexp(1.0, -x) <= fmax)
    assert np.all(a * np.ldexp(1.0, -(x - 1)) > fmax)
    # exactly on the boundary the scaled maximum is the largest finite value itself
    xe = F.e8m0_exponent(edge, name, "ceil")
    assert np.all(edge * np.ldexp(1.0, -xe) == fmax)


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_e8m0_ceil_vs_floor(name):
    """The rules differ by one exactly when the significand of a exceeds 1.75."""
    rng = np.random.default_rng(4)
    a = np.exp(rng.uniform(-60, 60, 100000))
    xf = F.e8m0_exponent(a, name)
    xc = F.e8m0_exponent(a, name, "ceil")
    m, _ = np.frexp(a)                       # a = m * 2^e, m in [0.5, 1)
    assert np.array_equal(xc - xf, (2.0 * m > 1.75).astype(np.int64))
    assert int(F.e8m0_exponent(np.array([0.0]), name, "ceil")[0]) == -127
    assert int(F.e8m0_exponent(np.array([1e300]), name, "ceil")[0]) == 127


def test_mx_ceil_rule_never_saturates():
    """Under the ceil rule every scaled element is within the finite range before rounding,
    so no code is produced by saturation: the codes equal the unclamped nearest rounding."""
    from oracle.norm import mx_quantize_rows
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 96)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    for name in ("e4m3", "e5m2"):
        fmt = F.FORMATS[name]
        codes, scales = mx_quantize_rows(v, name, rule="ceil")
        x = scales.astype(np.int64) - 127
        y32 = F.to_f32(v)
        for b in range(3):
            s = y32[:, 32 * b:32 * b + 32] * np.ldexp(1.0, -x[:, b])[:, None]
            assert np.all(np.abs(s) <= fmt.max_finite)
            assert np.array_equal(codes[:, 32 * b:32 * b + 32], F.fp8_quantize(s, fmt))
