"""GPU: random shapes and options against the oracle, a CU margin, a busy second stream and many
repeats.

* Property-based cases (hypothesis, derandomised so every run draws the same cases): random
  rows and hidden sizes (multiples of 8), input / weight dtypes, norm type, zero-centred gamma,
  scaling mode, FP8 format and quantised layout; the forward is checked against the oracle with
  the tolerances of tests/checks.py, and the backward of the same case as well.
* cu_margin > 0 shrinks the persistent grids (and the planner's resident-workgroup budget).
* A second stream keeps the GPU busy with matrix products while the library's kernels run:
  the results must not change (no kernel assumes that its whole grid is resident).
* 100 back-to-back calls of the cross-workgroup paths (delayed amax through the workspace,
  band kernel) give bitwise-identical results and leave the workspace header clean.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import workloads
from oracle import formats as F
import checks
from test_gpu_parity import EPS, T, assert_ws_clean, bits, env, gpu, ln_terms, oracle_bwd, oracle_fwd

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import rmsnorm_fp8_quantization_amd as nf  # noqa: E402

TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def check_forward(case, ref, out, norm, in_dt, w_dt, zc, scaling, fp8, layout, scale=None):
    t = ln_terms(case, ref, norm, w_dt, zc)
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                       out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    rowwise = layout != "colwise"
    colwise = layout != "rowwise"
    if scaling == "none":
        checks.check_hp(bits(out["y"]), ref["v"], in_dt, terms=t)
    elif scaling == "delayed":
        got = {"y": bits(out["y"]) if rowwise else None,
               "y_colwise": bits(out["y_colwise"]) if colwise else None,
               "scale_inv": out["scale_inv"].item() if rowwise else None,
               "colwise_scale_inv": out["colwise_scale_inv"].item() if colwise else None,
               "amax": out["amax"].item()}
        checks.check_delayed(got, ref["v"], scale, 0.0, fp8, rowwise=rowwise, colwise=colwise, terms=t)
    else:
        rule = "ceil" if scaling == "mxfp8_ceil" else "floor"
        if rowwise:
            checks.check_mx_rows(bits(out["y"]), bits(out["scale_inv"]), ref["v"], fp8, "mx rowwise",
                                 terms=t, rule=rule)
        if colwise:
            checks.check_mx_rows(bits(out["y_colwise"]), bits(out["colwise_scale_inv"]),
                                 np.ascontiguousarray(ref["v"].T), fp8, "mx colwise", terms=T(t), rule=rule)


@st.composite
def cases(draw):
    rows = draw(st.integers(1, 300))
    hidden = 8 * draw(st.integers(1, min(1536, 1_000_000 // (8 * rows))))
    norm = draw(st.sampled_from(["layernorm", "rmsnorm"]))
    in_dt = draw(st.sampled_from(["bf16", "f16", "f32"]))
    w_dt = draw(st.sampled_from(["f32", "bf16"]))
    zc = draw(st.booleans())
    scaling = draw(st.sampled_from(["none", "delayed", "mxfp8", "mxfp8_ceil"]))
    fp8 = draw(st.sampled_from(["e4m3", "e5m2"]))
    layout = "rowwise" if scaling == "none" else draw(st.sampled_from(["rowwise", "colwise", "rowwise_colwise"]))
    seed = draw(st.integers(0, 10_000))
    return rows, hidden, norm, in_dt, w_dt, zc, scaling, fp8, layout, seed


@settings(max_examples=40, derandomize=True, deadline=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(cases())
def test_random_cases_forward_and_backward(c):
    rows, hidden, norm, in_dt, w_dt, zc, scaling, fp8, layout, seed = c
    print(f"case rows={rows} hidden={hidden} {norm} in={in_dt} w={w_dt} zc={zc} {scaling} {fp8} {layout} "
          f"seed={seed}", flush=True)
    case = workloads.small_case(norm, rows, hidden, in_dt, w_dt, seed=seed, zero_centered_gamma=zc)
    ref = oracle_fwd(case, norm, in_dt, w_dt, zc)
    x, g, b, dy = gpu(case, "x", "gamma", "beta", "dy")
    kw = dict(norm=norm, eps=EPS, zero_centered_gamma=zc)
    scale = None
    if scaling == "delayed":
        fmax = F.FORMATS[fp8].max_finite
        scale = float(np.float32(fmax) / np.float32(np.max(np.abs(ref["v"])) / 2))
        kw.update(scaling="delayed", fp8=fp8, layout=layout, scale=torch.tensor([scale], device="cuda"),
                  amax=torch.zeros(1, device="cuda"))
    elif scaling != "none":
        kw.update(scaling=scaling, fp8=fp8, layout=layout)
    out = nf.fwd(x, g, b, **kw)
    check_forward(case, ref, out, norm, in_dt, w_dt, zc, scaling, fp8, layout, scale)
    # the backward of the same case, from the GPU's own statistics
    if hidden <= 16384:
        refb = oracle_bwd(case, norm, in_dt, w_dt, zc, ref)
        d = nf.bwd(dy, x, out["mu"], out["rsigma"], g, norm=norm, zero_centered_gamma=zc)
        checks.check_dx(bits(d["dx"]), refb["dx"], in_dt)
        checks.check_wgrad(bits(d["dgamma"]) if w_dt != "f32" else d["dgamma"].cpu().numpy(), refb["dgamma"], w_dt)
        if norm == "layernorm":
            checks.check_wgrad(bits(d["dbeta"]) if w_dt != "f32" else d["dbeta"].cpu().numpy(), refb["dbeta"],
                               w_dt, what="dbeta")
    assert_ws_clean()


@pytest.mark.parametrize("margin", [1, 64, 200])
@pytest.mark.parametrize("path", ["row", "tiles", "band"])
def test_cu_margin(margin, path):
    case = workloads.small_case("rmsnorm", 2048, 2048, "bf16", "f32", seed=margin)
    ref = oracle_fwd(case, "rmsnorm", "bf16", "f32", False)
    x, g, dy = gpu(case, "x", "gamma", "dy")
    scale = float(np.float32(448.0) / np.float32(np.max(np.abs(ref["v"]))))
    kw = dict(norm="rmsnorm", eps=EPS, cu_margin=margin)
    layout = "rowwise" if path == "row" else "rowwise_colwise"
    kw.update(scaling="delayed", fp8="e4m3", layout=layout, scale=torch.tensor([scale], device="cuda"),
              amax=torch.zeros(1, device="cuda"))
    with env(NORMFP8_COL_KERNEL=0 if path == "band" else 1):
        out = nf.fwd(x, g, None, **kw)
    check_forward(case, ref, out, "rmsnorm", "bf16", "f32", False, "delayed", "e4m3", layout, scale)
    refb = oracle_bwd(case, "rmsnorm", "bf16", "f32", False, ref)
    d = nf.bwd(dy, x, None, out["rsigma"], g, norm="rmsnorm", cu_margin=margin)
    checks.check_dx(bits(d["dx"]), refb["dx"], "bf16")
    checks.check_wgrad(d["dgamma"].cpu().numpy(), refb["dgamma"])
    assert_ws_clean()


def test_busy_second_stream():
    """Matrix products on a second stream occupy CUs while every forward path and the backward
    run on the default stream; results equal those of an idle GPU, bit for bit."""
    case = workloads.small_case("layernorm", 4096, 4096, "bf16", "f32", seed=77)
    x, g, b, dy = gpu(case, "x", "gamma", "beta", "dy")
    scale = torch.tensor([20.0], device="cuda")

    def run():
        outs = []
        outs += list(nf.fwd(x, g, b, norm="layernorm").values())
        o = nf.fwd(x, g, b, norm="layernorm", scaling="delayed", layout="rowwise_colwise", scale=scale,
                   amax=torch.zeros(1, device="cuda"))
        outs += list(o.values())
        with env(NORMFP8_COL_KERNEL=0):
            outs += list(nf.fwd(x, g, b, norm="layernorm", scaling="mxfp8", layout="rowwise_colwise").values())
        f = nf.fwd(x, g, b, norm="layernorm")
        outs += list(nf.bwd(dy, x, f["mu"], f["rsigma"], g, norm="layernorm").values())
        return [t.clone() for t in outs if t is not None]

    idle = run()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    a = torch.randn(4096, 4096, device="cuda")
    with torch.cuda.stream(side):
        busy_out = [a @ a for _ in range(40)]
    busy = run()
    torch.cuda.synchronize()
    del busy_out
    assert len(idle) == len(busy)
    for i, (u, v) in enumerate(zip(idle, busy)):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), f"output {i} differs under load"
    assert_ws_clean()


@pytest.mark.parametrize("path", ["tiles", "band"])
def test_hundred_repeats_bitwise(path):
    case = workloads.small_case("rmsnorm", 1000, 3072, "bf16", "f32", seed=9)
    x, g = gpu(case, "x", "gamma")
    scale = torch.tensor([30.0], device="cuda")
    first = None
    with env(NORMFP8_COL_KERNEL=0 if path == "band" else 1):
        for i in range(100):
            o = nf.fwd(x, g, None, norm="rmsnorm", scaling="delayed", layout="rowwise_colwise", scale=scale,
                       amax=torch.zeros(1, device="cuda"))
            cur = [o["y"], o["y_colwise"], o["amax"], o["rsigma"]]
            if first is None:
                first = [t.clone() for t in cur]
            else:
                for u, v in zip(first, cur):
                    assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), f"call {i} differs"
    assert_ws_clean()
