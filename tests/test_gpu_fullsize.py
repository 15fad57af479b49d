"""GPU parity at the benchmark workloads' full sizes, in the launch configuration bench.py times.

Row-local outputs (y, FP8 codes, MXFP8 blocks, mu, rsigma, dx) are checked on sampled rows
(or sampled 32-row bands for columnwise MXFP8) that the oracle computes one by one; tensor-wide
results (amax, dgamma, dbeta) are checked against the oracle streamed over every row.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import checks

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import rmsnorm_fp8_quantization_amd as nf  # noqa: E402

CHUNK = 1024


def npb(t):
    return W.to_numpy_bits(t.cpu() if t.is_cuda else t)


def oracle_rows(w, xb, g, b, rows):
    return oracle.forward_stored(xb[rows], g, b, norm=w.norm, eps=w.eps, in_dtype=w.in_dtype,
                                 w_dtype=w.w_dtype, zero_centered_gamma=w.zero_centered_gamma)


def oracle_stream(w, xb, g, b, dyb=None, resb=None):
    """Stats of every row, max |v| and (with dy) the weight gradients, chunk by chunk."""
    n = xb.shape[0]
    mu = np.zeros(n) if w.norm == "layernorm" else None
    rs = np.zeros(n)
    amax = 0.0
    dg = np.zeros(w.hidden)
    db = np.zeros(w.hidden) if w.norm == "layernorm" else None
    for r0 in range(0, n, CHUNK):
        sl = slice(r0, min(n, r0 + CHUNK))
        f = oracle_rows(w, xb, g, b, sl)
        rs[sl] = f["rsigma"]
        if mu is not None:
            mu[sl] = f["mu"]
        amax = max(amax, float(np.max(np.abs(f["v"]))))
        if dyb is not None:
            bw = oracle.backward_stored(dyb[sl], xb[sl], f["mu"], f["rsigma"], g, norm=w.norm,
                                        in_dtype=w.in_dtype, w_dtype=w.w_dtype,
                                        zero_centered_gamma=w.zero_centered_gamma,
                                        residual_dy=resb[sl] if resb is not None else None)
            dg += bw["dgamma"]
            if db is not None:
                db += bw["dbeta"]
    return {"mu": mu, "rsigma": rs, "amax": amax, "dgamma": dg, "dbeta": db}


def ln_terms(v, mu, rs, g, b):
    """|xhat * g| + |mu * rsigma * g| + |beta| per element: the magnitudes of the terms whose
    binary32 sum gives a LayerNorm y (the cancellation allowance of the checks)."""
    beta = oracle.decode_storage(b, "f32")[None, :]
    gam = oracle.decode_storage(g, "f32")[None, :]
    return np.abs(v - beta) + np.abs(mu[:, None] * rs[:, None] * gam) + np.abs(beta)


def sample_rows(n, k=48, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(k, n), replace=False)]))


def test_rms_f32_256x1024_fwd_bwd_whole_tensor():
    w = W.WORKLOADS["rms_f32_256x1024"]
    h = W.make_inputs(w)
    xb, g, dyb = npb(h["x"]), npb(h["gamma"]), npb(h["dy"])
    ref = oracle_rows(w, xb, g, None, slice(None))
    x, gg, dy = h["x"].cuda(), h["gamma"].cuda(), h["dy"].cuda()
    f = nf.fwd(x, gg, None, norm="rmsnorm", eps=w.eps)
    checks.check_stats(None, f["rsigma"].cpu().numpy(), None, ref["rsigma"])
    checks.check_hp(f["y"].cpu().numpy(), ref["v"], "f32")
    rb = oracle.backward_stored(dyb, xb, None, ref["rsigma"], g, norm="rmsnorm", in_dtype="f32", w_dtype="f32")
    d = nf.bwd(dy, x, None, torch.tensor(ref["rsigma"], dtype=torch.float32, device="cuda"), gg, norm="rmsnorm")
    checks.check_dx(d["dx"].cpu().numpy(), rb["dx"], "f32")
    checks.check_wgrad(d["dgamma"].cpu().numpy(), rb["dgamma"])


def test_ln_bf16_16384x4096_fwd_bwd():
    w = W.WORKLOADS["ln_bf16_16384x4096"]
    h = W.make_inputs(w)
    xb, g, b, dyb = npb(h["x"]), npb(h["gamma"]), npb(h["beta"]), npb(h["dy"])
    x, gg, bb, dy = (h[k].cuda() for k in ("x", "gamma", "beta", "dy"))
    f = nf.fwd(x, gg, bb, norm="layernorm", eps=w.eps)
    rows = sample_rows(w.rows)
    ref = oracle_rows(w, xb, g, b, rows)
    checks.check_stats(f["mu"].cpu().numpy()[rows], f["rsigma"].cpu().numpy()[rows], ref["mu"], ref["rsigma"])
    checks.check_hp(npb(f["y"])[rows], ref["v"], "bf16", terms=ln_terms(ref["v"], ref["mu"], ref["rsigma"], g, b))
    full = oracle_stream(w, xb, g, b, dyb)
    mu = torch.tensor(full["mu"], dtype=torch.float32, device="cuda")
    rs = torch.tensor(full["rsigma"], dtype=torch.float32, device="cuda")
    d = nf.bwd(dy, x, mu, rs, gg, norm="layernorm")
    rb = oracle.backward_stored(dyb[rows], xb[rows], full["mu"][rows], full["rsigma"][rows], g, norm="layernorm",
                                in_dtype="bf16", w_dtype="f32")
    checks.check_dx(npb(d["dx"])[rows], rb["dx"], "bf16")
    checks.check_wgrad(d["dgamma"].cpu().numpy(), full["dgamma"])
    checks.check_wgrad(d["dbeta"].cpu().numpy(), full["dbeta"], what="dbeta")


def test_rms_delayed_e4m3_32768x8192_rowwise_colwise():
    w = W.WORKLOADS["rms_bf16_32768x8192_delayed_e4m3"]
    h = W.make_inputs(w)
    prior = npb(W.make_inputs(w, prior=True)["x"])
    xb, g = npb(h["x"]), npb(h["gamma"])
    prior_amax = oracle_stream(w, prior, g, None)["amax"]          # previous step's amax
    scale = float(np.float32(448.0) / np.float32(prior_amax))
    x, gg = h["x"].cuda(), h["gamma"].cuda()
    out = nf.fwd(x, gg, None, norm="rmsnorm", eps=w.eps, scaling="delayed", fp8="e4m3",
                 scale=torch.tensor([scale], device="cuda"), amax=torch.zeros(1, device="cuda"),
                 layout="rowwise_colwise")
    full = oracle_stream(w, xb, g, None)
    rows = sample_rows(w.rows)
    ref = oracle_rows(w, xb, g, None, rows)
    got = {"y": npb(out["y"])[rows], "y_colwise": npb(out["y_colwise"])[:, rows],
           "scale_inv": out["scale_inv"].item(), "colwise_scale_inv": out["colwise_scale_inv"].item(),
           "amax": out["amax"].item()}
    # amax over the whole tensor: check it separately from the sampled rows' codes
    assert abs(got["amax"] - full["amax"]) <= 1e-6 * full["amax"]
    got["amax"] = float(np.max(np.abs(ref["v"])))
    checks.check_delayed(got, ref["v"], scale, 0.0, "e4m3", rowwise=True, colwise=True)
    checks.check_stats(None, out["rsigma"].cpu().numpy(), None, full["rsigma"])
    # one scale for the whole tensor: every columnwise code is the transposed rowwise code
    assert torch.equal(out["y_colwise"], out["y"].t().contiguous())
    assert nf.workspace_check() == 0


def test_rms_mxfp8_e4m3_16384x12288_rowwise_colwise():
    w = W.WORKLOADS["rms_bf16_16384x12288_mxfp8_e4m3"]
    h = W.make_inputs(w)
    xb, g = npb(h["x"]), npb(h["gamma"])
    x, gg = h["x"].cuda(), h["gamma"].cuda()
    out = nf.fwd(x, gg, None, norm="rmsnorm", eps=w.eps, zero_centered_gamma=True, scaling="mxfp8",
                 fp8="e4m3", layout="rowwise_colwise")
    yr, sr = npb(out["y"]), npb(out["scale_inv"])
    yc, sc = npb(out["y_colwise"]), npb(out["colwise_scale_inv"])
    rng = np.random.default_rng(1)
    bands = np.unique(np.concatenate([[0, w.rows // 32 - 1], rng.choice(w.rows // 32, 6, replace=False)]))
    boundary = 0
    for band in bands:
        rows = slice(32 * band, 32 * band + 32)
        ref = oracle_rows(w, xb, g, None, rows)
        print(f"band {band}", flush=True)
        checks.check_stats(None, out["rsigma"].cpu().numpy()[rows], None, ref["rsigma"])
        boundary += checks.check_mx_rows(yr[rows], sr[rows], ref["v"], "e4m3", "mx rowwise")["boundary_blocks"]
        boundary += checks.check_mx_rows(yc[:, rows], sc[:, band:band + 1], np.ascontiguousarray(ref["v"].T),
                                         "e4m3", "mx colwise")["boundary_blocks"]
    print(f"E8M0 power-of-two boundary blocks in the sample: {boundary}")
    assert nf.workspace_check() == 0


def test_ln_bf16_1024x65536_split_rows():
    w = W.WORKLOADS["ln_bf16_1024x65536"]
    h = W.make_inputs(w)
    xb, g, b = npb(h["x"]), npb(h["gamma"]), npb(h["beta"])
    x, gg, bb = h["x"].cuda(), h["gamma"].cuda(), h["beta"].cuda()
    out = nf.fwd(x, gg, bb, norm="layernorm", eps=w.eps)
    rows = sample_rows(w.rows, k=24)
    ref = oracle_rows(w, xb, g, b, rows)
    checks.check_stats(out["mu"].cpu().numpy()[rows], out["rsigma"].cpu().numpy()[rows], ref["mu"],
                       ref["rsigma"])
    checks.check_hp(npb(out["y"])[rows], ref["v"], "bf16", terms=ln_terms(ref["v"], ref["mu"], ref["rsigma"], g, b))
    assert nf.workspace_check() == 0


def test_rms_bwd_add_32768x8192():
    w = W.WORKLOADS["rms_bf16_32768x8192_bwd_add"]
    h = W.make_inputs(w)
    xb, g, dyb, rb_ = npb(h["x"]), npb(h["gamma"]), npb(h["dy"]), npb(h["residual_dy"])
    full = oracle_stream(w, xb, g, None, dyb, rb_)
    x, gg, dy, res = (h[k].cuda() for k in ("x", "gamma", "dy", "residual_dy"))
    rs = torch.tensor(full["rsigma"], dtype=torch.float32, device="cuda")
    d = nf.bwd_add(dy, x, res, rs, gg)
    rows = sample_rows(w.rows)
    ref = oracle.backward_stored(dyb[rows], xb[rows], None, full["rsigma"][rows], g, norm="rmsnorm",
                                 in_dtype="bf16", w_dtype="f32", residual_dy=rb_[rows])
    checks.check_dx(npb(d["dx"])[rows], ref["dx"], "bf16")
    checks.check_wgrad(d["dgamma"].cpu().numpy(), full["dgamma"])
