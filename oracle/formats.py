"""Number formats of the normalisation oracle, written as plain float64 definitions.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in ``__graft_entry__``
and the CPU-baseline leg of ``bench.py`` may import anything under ``oracle/``.
The HIP library and its Python binding never do; they share no code, table or
constant with this package.

Sources of the format facts (the normalisation pages name the modes -- delayed
per-tensor scaling, MXFP8 block scaling, E4M3/E5M2 outputs -- but do not define
the encodings):
  * OCP 8-bit Floating Point Specification (OFP8), rev. 1.0: E4M3 has bias 7,
    no infinities, one NaN mantissa (S.1111.111) and largest finite 448;
    E5M2 has bias 15, IEEE-style inf/NaN and largest finite 57344; both have
    subnormals.
  * OCP Microscaling Formats (MX) Specification v1.0: the E8M0 shared scale is a
    bare biased exponent (bias 127, 0xFF = NaN); for a block with largest
    magnitude a the shared exponent is floor(log2 a) minus the element format's
    largest normal exponent (8 for E4M3, 15 for E5M2).
  * IEEE 754 binary32 / binary16 and bfloat16 (binary32 with the low 16 mantissa
    bits dropped) for the high-precision outputs.

Rounding reading: every rounding here is round-to-nearest, ties-to-even.  For
the FP8 outputs, finite values beyond the largest finite code saturate to it
(the pages do not say; saturation keeps outliers that exceed a delayed scale
finite).  Parity unpinned against the pages for the saturation choice.
"""
from __future__ import annotations

import numpy as np


class Format:
    """A binary floating-point format described by its field widths."""

    def __init__(self, name, exp_bits, mant_bits, bias, max_finite, overflow):
        self.name = name
        self.exp_bits = exp_bits
        self.mant_bits = mant_bits
        self.bias = bias
        self.emin = 1 - bias                  # exponent of the smallest normal number
        self.max_finite = float(max_finite)
        self.overflow = overflow              # "inf" (IEEE) or "saturate"

    def __repr__(self):
        return f"Format({self.name})"


FP32 = Format("f32", 8, 23, 127, (2.0 - 2.0 ** -23) * 2.0 ** 127, "inf")
BF16 = Format("bf16", 8, 7, 127, (2.0 - 2.0 ** -7) * 2.0 ** 127, "inf")
FP16 = Format("f16", 5, 10, 15, 65504.0, "inf")
E4M3 = Format("e4m3", 4, 3, 7, 448.0, "saturate")
E5M2 = Format("e5m2", 5, 2, 15, 57344.0, "saturate")

FORMATS = {f.name: f for f in (FP32, BF16, FP16, E4M3, E5M2)}

# largest normal exponent of the MX element formats (OCP MX v1.0, element types)
MX_EMAX = {"e4m3": 8, "e5m2": 15}


def floor_log2(a):
    """floor(log2 a) for finite a > 0, exactly (frexp splits a = m * 2**k, m in [0.5, 1))."""
    _, k = np.frexp(np.asarray(a, dtype=np.float64))
    return k.astype(np.int64) - 1


def round_nearest_even(v, fmt: Format):
    """Value of ``fmt`` nearest to each float64 ``v``; ties go to the even significand.

    Near |v| the representable values are the integer multiples of
    q = 2**(max(floor(log2|v|), emin) - mant_bits); |v|/q is exact, so the choice
    between its floor and ceiling is made exactly.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)
    e = np.where(a_f > 0, floor_log2(np.where(a_f > 0, a_f, 1.0)), fmt.emin)
    e = np.maximum(e, fmt.emin)
    q = np.ldexp(1.0, (e - fmt.mant_bits).astype(np.int64))
    n = a_f / q
    fl = np.floor(n)
    frac = n - fl
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(fl, 2.0) == 1.0))
    r = (fl + up) * q
    if fmt.overflow == "saturate":
        r = np.minimum(r, fmt.max_finite)
        r = np.where(np.isinf(a), fmt.max_finite, r)
    else:
        r = np.where(r > fmt.max_finite, np.inf, r)
        r = np.where(np.isinf(a), np.inf, r)
    r = np.where(np.isnan(a), np.nan, r)
    return np.copysign(r, v)


def fp8_encode(r, fmt: Format):
    """Bit pattern (uint8) of values already on the FP8 grid (output of round_nearest_even)."""
    r = np.asarray(r, dtype=np.float64)
    sign = np.where(np.signbit(r), 0x80, 0x00).astype(np.int64)
    a = np.abs(r)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    normal = a >= 2.0 ** fmt.emin
    e = np.where(normal, floor_log2(np.where(normal, a, 1.0)), fmt.emin)
    exp_field = np.where(normal, e + fmt.bias, 0)
    frac_scale = np.ldexp(1.0, (fmt.mant_bits - e).astype(np.int64))
    mant_field = np.where(normal, a * frac_scale - 2 ** fmt.mant_bits, a * frac_scale)
    code = sign | (exp_field.astype(np.int64) << fmt.mant_bits) | mant_field.astype(np.int64)
    nan_code = 0x7F
    code = np.where(nan, nan_code, code)
    return code.astype(np.uint8)


def fp8_decode(code, fmt: Format):
    """float64 value of each FP8 bit pattern."""
    c = np.asarray(code).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    E = (c >> fmt.mant_bits) & ((1 << fmt.exp_bits) - 1)
    M = c & ((1 << fmt.mant_bits) - 1)
    sub = M * 2.0 ** (fmt.emin - fmt.mant_bits)
    nor = (1.0 + M / 2.0 ** fmt.mant_bits) * np.ldexp(1.0, (E - fmt.bias).astype(np.int64))
    val = np.where(E == 0, sub, nor)
    top = (1 << fmt.exp_bits) - 1
    if fmt.name == "e4m3":
        val = np.where((E == top) & (M == (1 << fmt.mant_bits) - 1), np.nan, val)
    else:
        val = np.where((E == top) & (M == 0), np.inf, val)
        val = np.where((E == top) & (M != 0), np.nan, val)
    return s * val


def fp8_quantize(v, fmt: Format):
    """Saturating round-to-nearest-even of float64 values to FP8 codes."""
    return fp8_encode(round_nearest_even(v, fmt), fmt)


def e8m0_exponent(a, fp8_name: str, rule: str = "floor"):
    """Shared MX block exponent X for a block whose largest magnitude is ``a`` (float64).

    rule "floor" (the OCP MX rule): X = floor(log2 a) - emax(element).
    rule "ceil": the smallest X with a * 2**-X <= the element format's largest finite value
    (448 for E4M3, 57344 for E5M2), i.e. X = ceil(log2(a / max)), so no element of the block
    saturates.  Both largest values are 1.75 * 2**emax, so with a = m * 2**E (m in [1, 2))
    this is E - emax, plus one when m > 1.75.
    Either way X is clamped to the E8M0 range [-127, 127]; an all-zero block takes the
    smallest scale, X = -127.  The stored byte is X + 127.
    """
    a = np.asarray(a, dtype=np.float64)
    pos = a > 0
    safe = np.where(pos, a, 1.0)
    x = floor_log2(safe) - MX_EMAX[fp8_name]
    if rule == "ceil":
        m = safe / np.ldexp(1.0, floor_log2(safe))          # significand in [1, 2), exact
        x = x + (m > 1.75)
    elif rule != "floor":
        raise ValueError(f"unknown E8M0 rule {rule!r}")
    x = np.where(pos, x, -127)
    return np.clip(x, -127, 127).astype(np.int64)


# ----------------------------------------------------------------------------------------
# storage dtypes of the high-precision tensors
# ----------------------------------------------------------------------------------------

def decode_storage(arr, dtype: str):
    """Exact float64 values of a stored tensor (bf16 arrives as uint16 bit patterns)."""
    arr = np.asarray(arr)
    if dtype == "bf16":
        assert arr.dtype == np.uint16, arr.dtype
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        assert arr.dtype == np.float16, arr.dtype
        return arr.astype(np.float64)
    if dtype == "f32":
        assert arr.dtype == np.float32, arr.dtype
        return arr.astype(np.float64)
    raise ValueError(dtype)


def encode_storage(v, dtype: str):
    """Round float64 values once (nearest-even) to a storage dtype; bf16 as uint16 bits."""
    fmt = FORMATS[dtype]
    r = round_nearest_even(v, fmt)
    if dtype == "bf16":
        return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    if dtype == "f16":
        return r.astype(np.float16)       # exact: r is already a binary16 value
    return r.astype(np.float32)           # exact: r is already a binary32 value


def to_f32(v):
    """Round float64 to the nearest binary32 value (as float64), ties to even."""
    return round_nearest_even(v, FP32)
