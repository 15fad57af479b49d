"""Pins of the oracle's normalisation, epilogues and backward (CPU only).

Checks against: torch float64 layer_norm / rms_norm / var_mean and autograd
(library routines), hand-worked closed forms (tests/golden/worked_norm.txt),
closed-form invariants, brute-force Python loops on tiny inputs, and central
finite differences of the forward for the backward.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle import norm as N

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, mean=0.0, std=1.0):
    return np.random.default_rng(seed).normal(mean, std, size=shape)


# ------------------------------------------------------------------- forward statistics

def test_worked_examples_golden():
    vals = {}
    with open(os.path.join(GOLDEN, "worked_norm.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                kind, key, *nums = line.split()
                vals[(kind, key)] = [float(n) for n in nums]
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    g = np.ones(4)
    ln = N.forward(x, g, np.zeros(4), N.LAYERNORM, vals[("ln", "eps")][0], round_stats=False)
    assert ln["mu"][0] == pytest.approx(vals[("ln", "mu")][0], rel=1e-15)
    assert ln["rsigma"][0] == pytest.approx(vals[("ln", "rsigma")][0], rel=1e-14)
    assert np.allclose(ln["v"][0], vals[("ln", "y")], rtol=1e-14, atol=0)
    rms = N.forward(x, g, None, N.RMSNORM, vals[("rms", "eps")][0], round_stats=False)
    assert rms["mu"] is None
    assert rms["rsigma"][0] == pytest.approx(vals[("rms", "rsigma")][0], rel=1e-14)
    assert np.allclose(rms["v"][0], vals[("rms", "y")], rtol=1e-14, atol=0)


@pytest.mark.parametrize("h", [1, 7, 64, 1000])
def test_layernorm_stats_match_torch_var_mean(h):
    x = _rand((9, h), h, 0.5, 3.0)
    eps = 1e-5
    mu, rs = N.row_stats(x, N.LAYERNORM, eps, round_to_f32=False)
    var_t, mu_t = torch.var_mean(torch.from_numpy(x), dim=1, unbiased=False)
    assert np.allclose(mu, mu_t.numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(rs, 1.0 / np.sqrt(var_t.numpy() + eps), rtol=1e-13)
    # the stored statistics are those values rounded once to binary32
    mu32, rs32 = N.row_stats(x, N.LAYERNORM, eps)
    assert np.array_equal(mu32, mu.astype(np.float32).astype(np.float64))
    assert np.array_equal(rs32, rs.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("norm", [N.LAYERNORM, N.RMSNORM])
def test_values_match_torch_float64(norm):
    x = _rand((17, 333), 3, 0.5, 3.0)
    gamma = _rand(333, 4, 1.0, 0.1)
    beta = _rand(333, 5, 0.0, 0.1)
    eps = 1e-5
    out = N.forward(x, gamma, beta if norm == N.LAYERNORM else None, norm, eps, round_stats=False)
    xt = torch.from_numpy(x)
    if norm == N.LAYERNORM:
        ref = torch.nn.functional.layer_norm(xt, (333,), torch.from_numpy(gamma),
                                             torch.from_numpy(beta), eps)
    else:
        ref = torch.nn.functional.rms_norm(xt, (333,), torch.from_numpy(gamma), eps)
    assert np.allclose(out["v"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_constant_row_closed_forms():
    eps = 1e-3
    c = 2.75
    x = np.full((3, 10), c)
    beta = _rand(10, 1)
    out = N.forward(x, _rand(10, 2, 1.0, 0.1), beta, N.LAYERNORM, eps, round_stats=False)
    assert np.all(out["mu"] == c)
    assert np.allclose(out["rsigma"], eps ** -0.5, rtol=1e-15)
    assert np.array_equal(out["v"], np.broadcast_to(beta, (3, 10)))
    rms = N.forward(x, np.ones(10), None, N.RMSNORM, eps, round_stats=False)
    assert np.allclose(rms["rsigma"], (c * c + eps) ** -0.5, rtol=1e-15)


def test_hidden_one_layernorm_gives_beta():
    x = _rand((5, 1), 8, 3.0, 2.0)
    out = N.forward(x, np.array([1.7]), np.array([0.3]), N.LAYERNORM, 1e-5, round_stats=False)
    assert np.array_equal(out["v"], np.full((5, 1), 0.3))


def test_unit_weight_invariants():
    eps = 1e-2
    x = _rand((6, 257), 9, 0.5, 3.0)
    ln = N.forward(x, np.ones(257), np.zeros(257), N.LAYERNORM, eps, round_stats=False)
    var = x.var(axis=1)
    assert np.allclose(ln["v"].sum(axis=1), 0.0, atol=1e-11)
    assert np.allclose((ln["v"] ** 2).mean(axis=1), var / (var + eps), rtol=1e-13)
    rms = N.forward(x, np.ones(257), None, N.RMSNORM, eps, round_stats=False)
    ms = (x ** 2).mean(axis=1)
    assert np.allclose((rms["v"] ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-13)


def test_fp32_stats_error_bound():
    """With binary32 statistics the LayerNorm row sum is no longer zero, but it is
    bounded by what the rounding of mu alone can cause."""
    x = _rand((50, 4096), 10, 0.5, 3.0)
    out = N.forward(x, np.ones(4096), np.zeros(4096), N.LAYERNORM, 1e-5)
    mu64 = np.array([math.fsum(r) / 4096 for r in x])
    bound = 4096 * np.abs(mu64 - out["mu"]) * out["rsigma"] * (1 + 1e-6) + 1e-9
    assert np.all(np.abs(out["v"].sum(axis=1)) <= bound)


def test_zero_centered_gamma_is_one_plus_gamma():
    x = _rand((4, 64), 11)
    # gamma = 0 under zero-centring is the unit weight: compare with torch rms_norm (no weight)
    out = N.forward(x, np.zeros(64), None, N.RMSNORM, 1e-5, zero_centered_gamma=True,
                    round_stats=False)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), None, 1e-5).numpy()
    assert np.allclose(out["v"], ref, rtol=1e-13, atol=1e-13)
    gam = _rand(64, 12, 0.0, 0.05)
    a = N.forward(x, gam, None, N.RMSNORM, 1e-5, zero_centered_gamma=True)["v"]
    ref2 = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(gam + 1.0),
                                        1e-5).numpy()
    assert np.allclose(a, ref2, rtol=1e-6, atol=1e-6)      # binary32 stats vs float64 stats


# ------------------------------------------------------------------- FP8 epilogues

def test_delayed_amax_scale_inv_and_no_saturation_at_exact_scale():
    x = _rand((8, 96), 13)
    x[3, 5] = 25.0
    v = N.forward(x, _rand(96, 14, 1.0, 0.1), None, N.RMSNORM, 1e-5)["v"]
    amax_bf = 0.0
    for r in range(8):                       # brute force
        for c in range(96):
            amax_bf = max(amax_bf, abs(v[r, c]))
    scale = float(np.float32(448.0) / np.float32(amax_bf))
    out = N.delayed_epilogue(v, scale, 0.0, "e4m3", colwise=True)
    assert out["amax"] == amax_bf
    assert N.delayed_epilogue(v, scale, 1e6, "e4m3", False)["amax"] == 1e6    # max with input
    assert out["scale_inv"] == np.float32(1.0) / np.float32(scale)
    # the largest element lands on (or within rounding of) 448 and nothing exceeds it
    dec = F.fp8_decode(out["rowwise"], F.E4M3)
    assert np.nanmax(np.abs(dec)) == 448.0
    assert int(np.argmax(np.abs(dec))) == int(np.argmax(np.abs(v)))
    # colwise is the quantisation of the transpose
    assert out["colwise"].shape == (96, 8)
    assert np.array_equal(out["colwise"], out["rowwise"].T)


def test_delayed_scale_inv_known_values():
    assert N.delayed_epilogue(np.ones((1, 1)), 4.0, 0, "e4m3", False)["scale_inv"] == np.float32(0.25)
    si = N.delayed_epilogue(np.ones((1, 1)), 3.0, 0, "e4m3", False)["scale_inv"]
    assert np.float32(si).view(np.uint32) == 0x3EAAAAAB


def test_delayed_codes_bruteforce_small():
    """Per-element scalar recomputation: u = v * s (one product of the unrounded value and the
    binary32 scale), code = nearest finite E5M2 value by exhaustive search over the 256 codes
    (ties to the even code)."""
    v = _rand((3, 40), 15) * 3.0
    s = 1234.5
    codes = N.delayed_quantize(v, s, "e5m2")
    table = F.fp8_decode(np.arange(256), F.E5M2)
    fin = [c for c in range(256) if math.isfinite(table[c])]
    for r in range(3):
        for c in range(40):
            u = float(v[r, c]) * float(np.float32(s))
            u = max(-57344.0, min(57344.0, u))
            best = min(fin, key=lambda k: (abs(table[k] - u), k % 2, k))
            assert F.fp8_decode(np.array([codes[r, c]]), F.E5M2)[0] == table[best]


def test_mx_rowwise_bruteforce_small():
    v = _rand((2, 80), 16) * np.exp(_rand((2, 80), 17))    # H = 80: last block has 16 elements
    codes, scales = N.mx_quantize_rows(v, "e4m3")
    assert codes.shape == (2, 80) and scales.shape == (2, 3)
    table = F.fp8_decode(np.arange(256), F.E4M3)
    fin = [c for c in range(256) if math.isfinite(table[c])]
    for r in range(2):
        for b in range(3):
            blk = [float(t) for t in v[r, 32 * b:32 * b + 32]]
            a = max(abs(t) for t in blk)
            x = math.floor(math.log2(a)) - 8
            assert scales[r, b] == x + 127
            for j, t in enumerate(blk):
                u = max(-448.0, min(448.0, t * 2.0 ** (-x)))
                best = min(fin, key=lambda k: (abs(table[k] - u), k % 2, k))
                assert table[codes[r, 32 * b + j]] == table[best]


def test_mx_zero_block_and_colwise_layout():
    v = np.zeros((64, 32))
    v[:, 0] = np.arange(64) - 10.0
    out = N.mx_epilogue(v, "e4m3", colwise=True)
    assert out["colwise"].shape == (32, 64) and out["colwise_scale"].shape == (32, 2)
    assert np.all(out["colwise_scale"][1:] == 0) and np.all(out["colwise"][1:] == 0)
    # column 0: rows 0..31 hold -10..21 (amax 21 -> X = 4 - 8); rows 32..63 hold 22..53
    # (amax 53 -> X = 5 - 8)
    assert list(out["colwise_scale"][0]) == [127 - 4, 127 - 3]
    # rowwise: every row has a single non-zero element in block 0
    r5 = int(out["rowwise_scale"][5, 0])
    assert r5 == math.floor(math.log2(5.0)) - 8 + 127


def test_mx_colwise_rowmajor_bruteforce_small():
    """The columnwise output in the rowwise orientation, worked element by element along the
    columns of a small matrix (70 rows: the last block of each column has 6 rows)."""
    v = _rand((70, 3), 18) * np.exp(_rand((70, 3), 19))
    out = N.mx_epilogue(v, "e4m3", colwise=True, col_layout="rowmajor")
    codes, scales = out["colwise"], out["colwise_scale"]
    assert codes.shape == (70, 3) and scales.shape == (3, 3)
    table = F.fp8_decode(np.arange(256), F.E4M3)
    fin = [c for c in range(256) if math.isfinite(table[c])]
    for j in range(3):
        for b in range(3):
            blk = [float(t) for t in v[32 * b:32 * b + 32, j]]
            a = max(abs(t) for t in blk)
            x = math.floor(math.log2(a)) - 8
            assert scales[b, j] == x + 127
            for i, t in enumerate(blk):
                u = max(-448.0, min(448.0, t * 2.0 ** (-x)))
                best = min(fin, key=lambda k: (abs(table[k] - u), k % 2, k))
                assert table[codes[32 * b + i, j]] == table[best]


# ------------------------------------------------------------------- backward

def _loss(x, gamma, beta, dy, norm, eps):
    return float((dy * N.forward(x, gamma, beta, norm, eps, round_stats=False)["v"]).sum())


@pytest.mark.parametrize("norm", [N.LAYERNORM, N.RMSNORM])
@pytest.mark.parametrize("rows,h", [(1, 1), (2, 2), (1, 3), (3, 5), (2, 8), (1, 33)])
def test_backward_matches_central_finite_differences(norm, rows, h):
    eps = 1e-3
    x = _rand((rows, h), 100 + h, 0.5, 2.0)
    gamma = _rand(h, 200 + h, 1.0, 0.3)
    beta = _rand(h, 300 + h, 0.0, 0.3) if norm == N.LAYERNORM else None
    dy = _rand((rows, h), 400 + h)
    mu, rs = N.row_stats(x, norm, eps, round_to_f32=False)
    got = N.backward(dy, x, mu, rs, gamma, norm)

    def fd(fn, arr):
        out = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            hstep = 1e-6 * max(1.0, abs(arr[i]))
            a1 = arr.copy(); a1[i] += hstep
            a2 = arr.copy(); a2[i] -= hstep
            out[i] = (fn(a1) - fn(a2)) / (2 * hstep)
        return out

    dx = fd(lambda a: _loss(a, gamma, beta, dy, norm, eps), x)
    dg = fd(lambda a: _loss(x, a, beta, dy, norm, eps), gamma)
    scale = max(1.0, np.abs(dx).max())
    assert np.allclose(got["dx"], dx, rtol=1e-5, atol=1e-6 * scale)
    assert np.allclose(got["dgamma"], dg, rtol=1e-5, atol=1e-6 * max(1.0, np.abs(dg).max()))
    if norm == N.LAYERNORM:
        db = fd(lambda a: _loss(x, gamma, a, dy, norm, eps), beta)
        assert np.allclose(got["dbeta"], db, rtol=1e-5, atol=1e-6)
    else:
        assert got["dbeta"] is None


def _fd(fn, arr):
    out = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        hstep = 1e-6 * max(1.0, abs(arr[i]))
        a1 = arr.copy(); a1[i] += hstep
        a2 = arr.copy(); a2[i] -= hstep
        out[i] = (fn(a1) - fn(a2)) / (2 * hstep)
    return out


@pytest.mark.parametrize("norm", [N.LAYERNORM, N.RMSNORM])
@pytest.mark.parametrize("rows,h", [(1, 1), (2, 3), (3, 8), (1, 33)])
def test_zero_centered_backward_matches_finite_differences(norm, rows, h):
    """backward_stored with zero_centered_gamma against central differences of
    L = sum(dy * y) where y is the zero-centred forward (weight 1 + gamma) and gamma is the raw
    parameter ([XLA-Norm] Signature / I/O Contract: zero_centered_gamma is an input of the
    forward and of the backward). A backward that dropped the + 1 would use the weight gamma
    (about 0.05 here) instead of about 1, and fail by a factor of ~20."""
    eps = 1e-3
    f32 = lambda a: np.asarray(a, np.float32)  # stored float32 tensors, exact in float64
    x = f32(_rand((rows, h), 500 + h, 0.5, 2.0)).astype(np.float64)
    gamma = f32(_rand(h, 600 + h, 0.0, 0.05)).astype(np.float64)
    beta = f32(_rand(h, 700 + h, 0.0, 0.3)).astype(np.float64) if norm == N.LAYERNORM else None
    dy = f32(_rand((rows, h), 800 + h)).astype(np.float64)

    def loss(xa, ga, ba):
        v = N.forward(xa, ga, ba, norm, eps, zero_centered_gamma=True, round_stats=False)["v"]
        return float((dy * v).sum())

    mu, rs = N.row_stats(x, norm, eps, round_to_f32=True)
    got = N.backward_stored(f32(dy), f32(x), mu, rs, f32(gamma), norm=norm, in_dtype="f32", w_dtype="f32",
                            zero_centered_gamma=True)
    dx = _fd(lambda a: loss(a, gamma, beta), x)
    dg = _fd(lambda a: loss(x, a, beta), gamma)
    # binary32 statistics in the backward: ~1e-7 relative against the exact-statistics differences
    assert np.allclose(got["dx"], dx, rtol=1e-5, atol=1e-5 * max(1.0, np.abs(dx).max()))
    assert np.allclose(got["dgamma"], dg, rtol=1e-5, atol=1e-5 * max(1.0, np.abs(dg).max()))
    if norm == N.LAYERNORM:
        db = _fd(lambda a: loss(x, gamma, a), beta)
        assert np.allclose(got["dbeta"], db, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("norm", [N.LAYERNORM, N.RMSNORM])
def test_zero_centered_backward_is_backward_at_one_plus_gamma(norm):
    """backward(gamma, zero-centred) is bitwise backward(1 + gamma, plain) for weights whose
    1 + gamma is exact in float32 (multiples of 2^-10 below 1)."""
    h = 96
    x = np.asarray(_rand((5, h), 61, 0.5, 2.0), np.float32)
    dy = np.asarray(_rand((5, h), 62), np.float32)
    gamma = np.asarray(np.round(_rand(h, 63, 0.0, 0.05) * 1024) / 1024, np.float32)
    gamma1 = gamma + np.float32(1.0)
    assert np.array_equal(gamma1.astype(np.float64), gamma.astype(np.float64) + 1.0)
    mu, rs = N.row_stats(x.astype(np.float64), norm, 1e-5)
    kw = dict(norm=norm, in_dtype="f32", w_dtype="f32")
    zc = N.backward_stored(dy, x, mu, rs, gamma, zero_centered_gamma=True, **kw)
    plain = N.backward_stored(dy, x, mu, rs, gamma1, zero_centered_gamma=False, **kw)
    raw = N.backward_stored(dy, x, mu, rs, gamma, zero_centered_gamma=False, **kw)
    assert np.array_equal(zc["dx"], plain["dx"]) and np.array_equal(zc["dgamma"], plain["dgamma"])
    assert not np.allclose(zc["dx"], raw["dx"])       # the flag is not a no-op
    # dgamma does not depend on the weight (d(1 + gamma)/dgamma = 1): sum of dy * xhat
    assert np.array_equal(zc["dgamma"], raw["dgamma"])
    if norm == N.LAYERNORM:
        assert np.array_equal(zc["dbeta"], plain["dbeta"])


@pytest.mark.parametrize("norm", [N.LAYERNORM, N.RMSNORM])
def test_backward_matches_torch_autograd(norm):
    eps = 1e-5
    x = _rand((12, 200), 21, 0.5, 3.0)
    gamma = _rand(200, 22, 1.0, 0.1)
    beta = _rand(200, 23, 0.0, 0.1)
    dy = _rand((12, 200), 24)
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(gamma, requires_grad=True)
    bt = torch.tensor(beta, requires_grad=True)
    if norm == N.LAYERNORM:
        y = torch.nn.functional.layer_norm(xt, (200,), gt, bt, eps)
    else:
        y = torch.nn.functional.rms_norm(xt, (200,), gt, eps)
    y.backward(torch.from_numpy(dy))
    mu, rs = N.row_stats(x, norm, eps, round_to_f32=False)
    got = N.backward(dy, x, mu, rs, gamma, norm)
    assert np.allclose(got["dx"], xt.grad.numpy(), rtol=1e-11, atol=1e-11)
    assert np.allclose(got["dgamma"], gt.grad.numpy(), rtol=1e-11, atol=1e-11)
    if norm == N.LAYERNORM:
        assert np.allclose(got["dbeta"], bt.grad.numpy(), rtol=1e-11, atol=1e-11)


def test_backward_invariants():
    eps = 1e-2
    x = _rand((5, 123), 31, 0.5, 2.0)
    g = _rand(123, 32, 1.0, 0.2)
    dy = _rand((5, 123), 33)
    mu, rs = N.row_stats(x, N.LAYERNORM, eps, round_to_f32=False)
    ln = N.backward(dy, x, mu, rs, g, N.LAYERNORM)
    assert np.allclose(ln["dx"].sum(axis=1), 0.0, atol=1e-11)
    _, rs2 = N.row_stats(x, N.RMSNORM, eps, round_to_f32=False)
    rms = N.backward(dy, x, None, rs2, g, N.RMSNORM)
    ms = (x ** 2).mean(axis=1)
    w = dy * g
    lhs = (rms["dx"] * x).sum(axis=1)
    rhs = rs2 * eps / (ms + eps) * (w * x).sum(axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-12)


def test_backward_add_is_plain_backward_plus_residual():
    x = _rand((4, 50), 41)
    dy = _rand((4, 50), 42)
    res = _rand((4, 50), 43, 0.0, 0.5)
    g = _rand(50, 44, 1.0, 0.1)
    _, rs = N.row_stats(x, N.RMSNORM, 1e-5)
    plain = N.backward(dy, x, None, rs, g, N.RMSNORM)
    fused = N.backward_add(dy, x, rs, g, res)
    assert np.array_equal(fused["dx"] - plain["dx"], res) or np.allclose(
        fused["dx"] - plain["dx"], res, rtol=0, atol=1e-15)
    assert np.array_equal(fused["dgamma"], plain["dgamma"])


def test_dgamma_dbeta_bruteforce():
    x = _rand((6, 5), 51)
    dy = _rand((6, 5), 52)
    g = _rand(5, 53, 1.0, 0.1)
    mu, rs = N.row_stats(x, N.LAYERNORM, 1e-5)
    out = N.backward(dy, x, mu, rs, g, N.LAYERNORM)
    for j in range(5):
        dg = sum(dy[r, j] * (x[r, j] - mu[r]) * rs[r] for r in range(6))
        db = sum(dy[r, j] for r in range(6))
        assert out["dgamma"][j] == pytest.approx(dg, rel=1e-13, abs=1e-14)
        assert out["dbeta"][j] == pytest.approx(db, rel=1e-13, abs=1e-14)


def test_stored_wrappers_decode_inputs():
    import workloads
    case = workloads.small_case("layernorm", 4, 64, "bf16", "f32", seed=3)
    xb = workloads.to_numpy_bits(case["x"])
    out = N.forward_stored(xb, case["gamma"].numpy(), case["beta"].numpy(), norm="layernorm",
                           eps=1e-5, in_dtype="bf16", w_dtype="f32")
    ref = torch.nn.functional.layer_norm(case["x"].double(), (64,), case["gamma"].double(),
                                         case["beta"].double(), float(np.float32(1e-5)))
    assert np.allclose(out["v"], ref.numpy(), rtol=1e-6, atol=1e-6)
