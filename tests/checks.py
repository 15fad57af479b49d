"""Element-wise acceptance checks of GPU outputs against the CPU oracle.

Tolerances (written here, used by every parity test):
  mu              |g - v| / max(|v|, 1e-3 * sigma_row) <= 1e-5
  rsigma          |g - v| / v <= 1e-5
  bf16 / f16 y    ordered-bit distance to the nearest-even rounding of v <= 1 ulp (where
                  LayerNorm's terms cancel: within half an ulp plus the binary32 evaluation
                  bound 2^-21 * (|xhat*g| + |mu*rsigma*g| + |beta|))
  f32 y, f32 dx   |g - v| / max(|v|, rms_row(v)) <= 1e-5
  FP8 codes       ordered code distance <= 1; at most 0.1% of elements differ; each
                  differing element's exact scaled value lies within 1e-5 (relative) of
                  the midpoint between the two codes' values, i.e. on a rounding boundary
                  (LayerNorm: plus the binary32 evaluation bound 2^-21 * terms, scaled like
                  the value, where terms = |xhat*g| + |mu*rsigma*g| + |beta| -- the same
                  allowance as for bf16 outputs, since the code is decided from a binary32 y)
  E8M0 scales     bit-exact against the exponent of the float64 block maximum, except blocks
                  whose float64 maximum lies within 2^-19 (relative) of a decision boundary of
                  the exponent rule (a power of two; 1.75 times a power of two for the round-up
                  rule), where the kernel's binary32 maximum may fall on either side: there
                  either neighbouring exponent is accepted and the block's codes are checked
                  under the GPU's exponent
  allowances      elements (or blocks) that pass only through an allowance -- the LayerNorm
                  cancellation slack of 16-bit y and FP8 codes, the E8M0 boundary window --
                  are counted, reported, and bounded: at most max(1, 1e-4 * n) of n
  amax            |g - v| / v <= 1e-6
  scale_inv       bit-exact
  bf16 / f16 dx   (|g - v| - half_ulp(v)) / max(|v|, rms_row(v)) <= 2e-3: the error beyond
                  the output's own nearest rounding (bf16 alone can be 2^-8 relative away
                  from v just above a power of two, more than 2e-3); for rows of fewer than
                  8 elements, whose summands cancel, the denominator also takes the summands'
                  magnitude rsigma * |dy * g|
  dgamma, dbeta   |g - v| / max(|v|, rms(v)) <= 1e-4
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle import formats as F

# e8m0_window: the binary32 kernel reaches a block maximum through a tree sum of squares over
# the row ((log2 H + 1) * 2^-24 relative at H = 12288 is ~9e-7, half of it in rsigma) and
# three roundings of y, ~2^-20 together; 2^-19 bounds it.
TOL = dict(mu=1e-5, rsigma=1e-5, f32=1e-5, dx16=2e-3, wgrad=1e-4, amax=1e-6, fp8_frac=1e-3,
           fp8_tau=1e-5, e8m0_window=2.0 ** -19, allowance_frac=1e-4)


def allowance_budget(n: int) -> int:
    """Most elements (or blocks) of n that may pass only through an allowance."""
    return max(1, int(TOL["allowance_frac"] * n))


class Report(dict):
    """Counts kept by a check (printed by tests on failure)."""


def _ordered(bits: np.ndarray, nbits: int) -> np.ndarray:
    """Map sign-magnitude float bit patterns to integers ordered like the values."""
    b = bits.astype(np.int64)
    sign = 1 << (nbits - 1)
    mag = b & (sign - 1)
    return np.where(b & sign, -mag, mag)


def check_stats(mu_g, rs_g, mu_ref, rs_ref, rows_sigma=None):
    rs_g = np.asarray(rs_g, np.float64)
    err = np.abs(rs_g - rs_ref) / rs_ref
    assert np.all(err <= TOL["rsigma"]), f"rsigma max rel err {err.max():.3e}"
    if mu_ref is not None:
        sig = rows_sigma if rows_sigma is not None else 1.0 / rs_ref
        den = np.maximum(np.abs(mu_ref), 1e-3 * sig)
        e2 = np.abs(np.asarray(mu_g, np.float64) - mu_ref) / den
        assert np.all(e2 <= TOL["mu"]), f"mu max rel err {e2.max():.3e}"


def check_hp(y_g: np.ndarray, v: np.ndarray, dtype: str, what="y", terms=None, aggregate=False):
    """High-precision output (f32 / f16 / bf16 storage) against unrounded v.

    16-bit outputs: at most 1 ulp from the nearest-even rounding of v. Where y is the small
    difference of larger terms (LayerNorm: x * rsigma * g, the mean's share and beta cancelling;
    `terms` holds |xhat * g| + |mu * rsigma * g| + |beta|), a binary32 evaluation (with binary32
    statistics) is only accurate to a few binary32 ulps of
    those terms, which can exceed one ulp of the small result: such elements pass when
    |g - v| <= half an ulp of v + 2^-21 * terms (eight binary32 roundings of the terms)."""
    if dtype == "f32":
        g = np.asarray(y_g, np.float64)
        rms = np.sqrt(np.mean(v * v, axis=-1, keepdims=True))
        den = np.maximum(np.abs(v), rms)
        err = np.abs(g - v) / np.where(den > 0, den, 1.0)
        assert np.all(err <= TOL["f32"]), f"{what}: max rel err {err.max():.3e}"
        return Report(max_err=float(err.max()), n=int(g.size), cancellation=0, off_by_one=0)
    ref = oracle.encode_storage(v, dtype)
    raw = np.asarray(y_g).view(np.uint16)
    d = np.abs(_ordered(raw, 16) - _ordered(np.asarray(ref).view(np.uint16), 16))
    far = d > 1
    n_cancel = 0
    if far.any() and terms is not None:
        g = F.decode_storage(raw if dtype == "bf16" else raw.view(np.float16), dtype)
        bound = half_ulp(v, dtype) + 2.0 ** -21 * np.asarray(terms, np.float64)
        ok = np.abs(g - v) <= bound
        n_cancel = int((far & ok).sum())
        far = far & ~ok
    assert not far.any(), f"{what}: {int(far.sum())} elements more than 1 ulp off"
    assert aggregate or n_cancel <= allowance_budget(d.size), \
        f"{what}: {n_cancel} of {d.size} elements pass only through the cancellation allowance"
    return Report(off_by_one=int((d == 1).sum()), cancellation=n_cancel, n=int(d.size))


def check_fp8(codes_g: np.ndarray, codes_ref: np.ndarray, u_exact: np.ndarray, fp8: str, what="codes",
              slack=None, check_fraction=True):
    """FP8 codes: <= 1 code apart, every difference on a rounding boundary (within 1e-5
    relative, plus `slack`, an absolute allowance per element in scaled units), and <= 0.1 %
    differing (skipped with check_fraction=False when the caller checks the fraction over a
    whole tensor assembled from pieces). Returns the count of differing codes in `differ`."""
    fmt = F.FORMATS[fp8]
    cg = np.asarray(codes_g, np.uint8)
    cr = np.asarray(codes_ref, np.uint8)
    diff = cg != cr
    n = int(diff.sum())
    if n == 0:
        return Report(differ=0, slack=0)
    og = _ordered(cg.astype(np.int64), 8)
    orf = _ordered(cr.astype(np.int64), 8)
    dist = np.abs(og - orf)
    # +0 / -0 are the same value
    zero_pair = (F.fp8_decode(cg[diff], fmt) == 0) & (F.fp8_decode(cr[diff], fmt) == 0)
    far = ~((dist[diff] <= 1) | zero_pair)
    # LayerNorm (`slack` given): a value near zero is the binary32 sum of terms that cancel, and
    # where the code spacing is finer than that evaluation allowance (E5M2 near zero) the code
    # can be several steps off. Such a code passes when its value lies within the allowance plus
    # one code spacing of the exact scaled value; it counts against the same allowance budget.
    multi = np.zeros_like(far)
    if far.any() and slack is not None:
        vgf = F.fp8_decode(cg[diff][far], fmt)
        uf = np.clip(np.asarray(u_exact, np.float64)[diff][far], -fmt.max_finite, fmt.max_finite)
        ef = np.floor(np.log2(np.maximum(np.abs(vgf), 2.0 ** fmt.emin)))
        spacing = 2.0 ** (np.maximum(ef, fmt.emin) - fmt.mant_bits)
        within = np.abs(vgf - uf) <= np.asarray(slack, np.float64)[diff][far] + spacing
        fi = np.flatnonzero(far)
        multi[fi[within]] = True
        far[fi[within]] = False
    if far.any():
        idx = np.argwhere(diff)[far][:6]
        raise AssertionError(
            f"{what}: {int(far.sum())} codes more than one step apart at {idx.tolist()}: gpu "
            f"{[hex(int(cg[tuple(i)])) for i in idx]} oracle {[hex(int(cr[tuple(i)])) for i in idx]} "
            f"exact scaled {[float(np.asarray(u_exact)[tuple(i)]) for i in idx]}")
    vg = F.fp8_decode(cg[diff], fmt)
    vr = F.fp8_decode(cr[diff], fmt)
    mid = 0.5 * (vg + vr)
    u = np.clip(np.asarray(u_exact, np.float64)[diff], -fmt.max_finite, fmt.max_finite)
    bound = TOL["fp8_tau"] * np.maximum(np.abs(u), 2.0 ** (fmt.emin - fmt.mant_bits))
    strict_ok = (np.abs(u - mid) <= bound) | zero_pair
    if slack is not None:
        bound = bound + np.asarray(slack, np.float64)[diff]
    ok = (np.abs(u - mid) <= bound) | zero_pair | multi
    n_slack = int((ok & ~strict_ok).sum())  # on a boundary only within the LayerNorm allowance
    if not np.all(ok):
        bad = ~ok
        raise AssertionError(
            f"{what}: {int(bad.sum())} differing codes not on a rounding boundary: at "
            f"{np.argwhere(diff)[bad][:4].tolist()} exact scaled {u[bad][:4]}, midpoint {mid[bad][:4]}, "
            f"allowed distance {bound[bad][:4]}")
    if check_fraction:
        frac = n / cg.size
        assert frac <= TOL["fp8_frac"], f"{what}: {n} of {cg.size} codes differ ({frac:.2e})"
        assert n_slack <= allowance_budget(cg.size), \
            f"{what}: {n_slack} of {cg.size} codes pass only through the cancellation allowance"
    return Report(differ=n, slack=n_slack)


def eval_slack(terms, factor):
    """Binary32 evaluation allowance 2^-21 * terms, in scaled units (None without terms)."""
    if terms is None:
        return None
    return 2.0 ** -21 * np.asarray(terms, np.float64) * factor


def check_delayed(out, v, scale, amax_in, fp8, rowwise=True, colwise=False, terms=None):
    """All delayed-scaling outputs against the oracle (v: float64 values [rows, hidden];
    terms: LayerNorm term magnitudes, see the module docstring)."""
    ref = oracle.delayed_epilogue(v, scale, amax_in, fp8, colwise)
    s32 = np.float64(np.float32(scale))
    u = v * s32
    slack = eval_slack(terms, s32)
    rep = Report()
    if rowwise:
        rep["row"] = check_fp8(out["y"], ref["rowwise"], u, fp8, "rowwise codes", slack)
        assert np.float32(out["scale_inv"]).view(np.uint32) == np.float32(ref["scale_inv"]).view(np.uint32)
    if colwise:
        rep["col"] = check_fp8(out["y_colwise"], ref["colwise"], np.ascontiguousarray(u.T), fp8, "colwise codes",
                               None if slack is None else np.ascontiguousarray(slack.T))
        assert np.float32(out["colwise_scale_inv"]).view(np.uint32) == np.float32(ref["scale_inv"]).view(np.uint32)
    a = float(out["amax"])
    assert abs(a - ref["amax"]) <= TOL["amax"] * ref["amax"], f"amax {a} vs {ref['amax']}"
    return rep


def check_mx_rows(codes_g, scales_g, v, fp8, what="mx", terms=None, rule="floor", aggregate=False):
    """MXFP8 blocks along the last axis of v (float64 [r, c]) against GPU codes / scale bytes
    (terms: LayerNorm term magnitudes laid out like v, see the module docstring; rule: the
    E8M0 exponent rule, whose decision boundaries are the powers of two for "floor" and
    1.75 times the powers of two for "ceil")."""
    fmt = F.FORMATS[fp8]
    v = np.asarray(v, np.float64)
    r, c = v.shape
    nb = -(-c // 32)
    codes_g = np.asarray(codes_g, np.uint8)
    scales_g = np.asarray(scales_g, np.uint8)
    assert scales_g.shape == (r, nb) and codes_g.shape == (r, c)
    boundary = 0
    differ = 0
    n_slack = 0
    for b in range(nb):
        sl = slice(32 * b, min(32 * b + 32, c))
        a64 = np.max(np.abs(v[:, sl]), axis=1)
        x_ref = F.e8m0_exponent(a64, fp8, rule)
        x_g = scales_g[:, b].astype(np.int64) - 127
        bad = x_g != x_ref
        if bad.any():
            # allowed only next to a decision boundary of the rule, and only by one step
            base = 1.75 if rule == "ceil" else 1.0
            k = np.floor(np.log2(np.where(a64 > 0, a64, 1.0) / base))
            lo_edge, hi_edge = base * 2.0 ** k, base * 2.0 ** (k + 1)
            near = (np.abs(a64 - lo_edge) <= TOL["e8m0_window"] * a64) | \
                   (np.abs(a64 - hi_edge) <= TOL["e8m0_window"] * a64)
            if not np.all(near[bad] & (np.abs(x_g - x_ref)[bad] == 1)):
                dist = np.minimum(np.abs(a64 - lo_edge), np.abs(a64 - hi_edge))[bad] / a64[bad]
                raise AssertionError(
                    f"{what} block {b}: {int(bad.sum())} E8M0 scales differ: rows {np.nonzero(bad)[0][:8]}, "
                    f"gpu X {x_g[bad][:8]}, oracle X {x_ref[bad][:8]}, block max {a64[bad][:8]}, "
                    f"relative distance to the rule's boundary {dist[:8]}")
            boundary += int(bad.sum())
        # reference codes under the GPU's exponent: one rounding of the float64 value
        u_exact = v[:, sl] * np.ldexp(1.0, -x_g)[:, None]
        ref_codes = F.fp8_quantize(u_exact, fmt)
        slack = None if terms is None else eval_slack(np.asarray(terms)[:, sl], np.ldexp(1.0, -x_g)[:, None])
        rb = check_fp8(codes_g[:, sl], ref_codes, u_exact, fp8, f"{what} block {b}", slack, check_fraction=False)
        differ += rb["differ"]
        n_slack += rb["slack"]
    rep = Report(boundary_blocks=boundary, differ=differ, slack=n_slack, blocks=r * nb, n=int(codes_g.size))
    if not aggregate:
        assert_mx_totals([rep], what)
    return rep


def assert_mx_totals(reports, what="mx"):
    """The tensor-wide bounds of check_mx_rows over reports of pieces of one tensor."""
    n = sum(r["n"] for r in reports)
    blocks = sum(r["blocks"] for r in reports)
    differ = sum(r["differ"] for r in reports)
    boundary = sum(r["boundary_blocks"] for r in reports)
    slack = sum(r["slack"] for r in reports)
    frac = differ / max(n, 1)
    assert frac <= TOL["fp8_frac"], f"{what}: {differ} of {n} codes differ ({frac:.2e})"
    assert boundary <= allowance_budget(blocks), \
        f"{what}: {boundary} of {blocks} E8M0 scales differ inside the boundary window"
    assert slack <= allowance_budget(n), f"{what}: {slack} of {n} codes pass only through the cancellation allowance"
    return Report(n=n, blocks=blocks, differ=differ, boundary_blocks=boundary, slack=slack)


def assert_fp8_totals(reports, n, what="codes"):
    """The tensor-wide bounds of check_fp8 over reports of n codes checked in pieces."""
    differ = sum(r["differ"] for r in reports)
    slack = sum(r["slack"] for r in reports)
    assert differ / max(n, 1) <= TOL["fp8_frac"], f"{what}: {differ} of {n} codes differ"
    assert slack <= allowance_budget(n), f"{what}: {slack} of {n} codes pass only through the cancellation allowance"
    return Report(n=n, differ=differ, slack=slack)


def assert_hp_totals(reports, what="y"):
    """The tensor-wide cancellation bound of check_hp over reports of pieces of one tensor."""
    n = sum(r["n"] for r in reports)
    cancel = sum(r["cancellation"] for r in reports)
    assert cancel <= allowance_budget(n), f"{what}: {cancel} of {n} elements pass only through the cancellation allowance"
    return Report(n=n, cancellation=cancel, off_by_one=sum(r["off_by_one"] for r in reports))


def half_ulp(v, dtype):
    """Half the spacing of the storage format around each |v| (the output rounding bound)."""
    fmt = F.FORMATS[dtype]
    a = np.abs(np.asarray(v, np.float64))
    e = np.where(a > 0, F.floor_log2(np.where(a > 0, a, 1.0)), fmt.emin)
    return np.ldexp(0.5, (np.maximum(e, fmt.emin) - fmt.mant_bits).astype(np.int64))


def check_dx(dx_g, v, dtype, terms=None):
    """dx against unrounded v: the error beyond the output's own nearest rounding (half an
    ulp of the storage format) must stay within the relative tolerance. terms (optional,
    laid out like v): the magnitude rsigma * |dy * g| of the summands of dx, for rows so short
    that the summands cancel (a row of one element has dx = rsigma * w * (1 - xhat^2), a
    difference of nearly equal binary32 values); the error is then measured against them."""
    g = np.asarray(dx_g, np.float64) if dtype == "f32" else F.decode_storage(np.asarray(dx_g), dtype)
    rms = np.sqrt(np.mean(v * v, axis=-1, keepdims=True))
    den = np.maximum(np.abs(v), rms)
    if terms is not None:
        den = np.maximum(den, np.asarray(terms, np.float64))
    excess = np.maximum(np.abs(g - v) - half_ulp(v, dtype), 0.0)
    err = excess / np.where(den > 0, den, 1.0)
    tol = TOL["f32"] if dtype == "f32" else TOL["dx16"]
    assert np.all(err <= tol), f"dx: max rel err beyond output rounding {err.max():.3e} (tol {tol})"
    return Report(max_err=float(err.max()))


def check_wgrad(g_gpu, v, dtype="f32", what="dgamma"):
    g = np.asarray(g_gpu, np.float64) if dtype == "f32" else F.decode_storage(np.asarray(g_gpu), dtype)
    rms = np.sqrt(np.mean(v * v))
    den = np.maximum(np.abs(v), rms if rms > 0 else 1.0)
    err = np.abs(g - v) / den
    tol = TOL["wgrad"] if dtype == "f32" else 2 ** -8
    assert np.all(err <= tol), f"{what}: max rel err {err.max():.3e}"
    return Report(max_err=float(err.max()))
