"""GPU: the general kernels -- hidden sizes that are not a multiple of 8, rows longer than the
row layouts, and tensors aligned only to their element size -- against the oracle.

The same checks (tests/checks.py) as the vector paths; the oracle has no notion of alignment or
strips, so these cases are pinned exactly like the others.
"""
import numpy as np
import pytest
import torch

import workloads
import checks
from test_gpu_parity import EPS, T, assert_ws_clean, bits, gpu, ln_terms, oracle_bwd, oracle_fwd
from test_gpu_stress import check_forward

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import rmsnorm_fp8_quantization_amd as nf  # noqa: E402

SHAPES = [(1, 1), (5, 3), (70, 7), (33, 100), (64, 1001), (9, 4100)]


def run_fwd(case, ref, norm, scaling, fp8, layout, zc=False):
    x, g, b = gpu(case, "x", "gamma", "beta")
    kw = dict(norm=norm, eps=EPS, zero_centered_gamma=zc)
    scale = None
    if scaling == "delayed":
        scale = float(np.float32(448.0) / np.float32(np.max(np.abs(ref["v"])) / 2))
        kw.update(scaling="delayed", fp8=fp8, layout=layout, scale=torch.tensor([scale], device="cuda"),
                  amax=torch.zeros(1, device="cuda"))
    elif scaling != "none":
        kw.update(scaling=scaling, fp8=fp8, layout=layout)
    return nf.fwd(x, g, b, **kw), scale


@pytest.mark.parametrize("rows,hidden", SHAPES)
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("scaling,layout", [("none", "rowwise"), ("delayed", "rowwise_colwise"),
                                            ("mxfp8", "rowwise_colwise"), ("mxfp8_ceil", "colwise_rowmajor"),
                                            ("delayed", "colwise")])
def test_general_hidden_forward(rows, hidden, norm, scaling, layout):
    case = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=rows * 3 + hidden)
    ref = oracle_fwd(case, norm, "bf16", "f32", False)
    out, scale = run_fwd(case, ref, norm, scaling, "e4m3", layout)
    lay = layout.replace("_rowmajor", "")
    if layout.endswith("_rowmajor"):   # compare in the transposed orientation the checks use
        out = dict(out)
        out["y_colwise"] = out["y_colwise"].T.contiguous()
        out["colwise_scale_inv"] = out["colwise_scale_inv"].T.contiguous()
    check_forward(case, ref, out, norm, "bf16", "f32", False, scaling, "e4m3", lay, scale)
    assert_ws_clean()


def dx_terms(case, ref_f, in_dt):
    """rsigma * |dy * g| per element (the summands' magnitude, see checks.check_dx)."""
    from test_gpu_parity import host_np
    from oracle import formats as F
    dy = F.decode_storage(host_np(case["dy"], in_dt), in_dt)
    g = F.decode_storage(host_np(case["gamma"], "f32"), "f32")[None, :]
    return np.asarray(ref_f["rsigma"])[:, None] * np.abs(dy * g)


@pytest.mark.parametrize("rows,hidden", SHAPES + [(3, 40000)])
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
def test_general_hidden_backward(rows, hidden, norm, in_dt):
    case = workloads.small_case(norm, rows, hidden, in_dt, "f32", seed=rows + hidden)
    ref_f = oracle_fwd(case, norm, in_dt, "f32", False)
    ref = oracle_bwd(case, norm, in_dt, "f32", False, ref_f)
    dy, x, g = gpu(case, "dy", "x", "gamma")
    mu = torch.tensor(ref_f["mu"], dtype=torch.float32, device="cuda") if norm == "layernorm" else None
    rs = torch.tensor(ref_f["rsigma"], dtype=torch.float32, device="cuda")
    out = nf.bwd(dy, x, mu, rs, g, norm=norm)
    checks.check_dx(bits(out["dx"]), ref["dx"], in_dt, terms=dx_terms(case, ref_f, in_dt) if hidden < 8 else None)
    checks.check_wgrad(out["dgamma"].cpu().numpy(), ref["dgamma"])
    if norm == "layernorm":
        checks.check_wgrad(out["dbeta"].cpu().numpy(), ref["dbeta"], what="dbeta")


@pytest.mark.parametrize("rows,hidden", [(40, 3), (64, 1001)])
def test_general_hidden_backward_add(rows, hidden):
    case = workloads.small_case("rmsnorm", rows, hidden, "bf16", "f32", seed=hidden)
    ref_f = oracle_fwd(case, "rmsnorm", "bf16", "f32", False)
    ref = oracle_bwd(case, "rmsnorm", "bf16", "f32", False, ref_f, add=True)
    dy, x, g, res = gpu(case, "dy", "x", "gamma", "residual_dy")
    rs = torch.tensor(ref_f["rsigma"], dtype=torch.float32, device="cuda")
    out = nf.bwd_add(dy, x, res, rs, g)
    checks.check_dx(bits(out["dx"]), ref["dx"], "bf16", terms=dx_terms(case, ref_f, "bf16") if hidden < 8 else None)
    checks.check_wgrad(out["dgamma"].cpu().numpy(), ref["dgamma"])


def offset_copy(t, elems=1):
    """A contiguous copy of t whose data starts `elems` elements past an aligned allocation."""
    buf = torch.empty(t.numel() + elems, dtype=t.dtype, device="cuda")
    v = buf[elems:].view(t.shape)
    v.copy_(t.cuda())
    return v


@pytest.mark.parametrize("scaling,layout", [("none", "rowwise"), ("mxfp8", "rowwise_colwise"),
                                            ("delayed", "rowwise_colwise")])
def test_element_aligned_tensors_forward(scaling, layout):
    """hidden a multiple of 8 but x starting 2 bytes past a 16-byte boundary: the general kernels
    serve it, and the results match the oracle (and the aligned call's)."""
    rows, hidden = 96, 1024
    case = workloads.small_case("layernorm", rows, hidden, "bf16", "f32", seed=12)
    ref = oracle_fwd(case, "layernorm", "bf16", "f32", False)
    xa = offset_copy(case["x"])
    assert xa.data_ptr() % 16 == 2
    g, b = gpu(case, "gamma", "beta")
    kw = dict(norm="layernorm", eps=EPS)
    scale = None
    if scaling == "delayed":
        scale = float(np.float32(448.0) / np.float32(np.max(np.abs(ref["v"]))))
        kw.update(scaling="delayed", layout=layout, scale=torch.tensor([scale], device="cuda"),
                  amax=torch.zeros(1, device="cuda"))
    elif scaling != "none":
        kw.update(scaling=scaling, layout=layout)
    out = nf.fwd(xa, g, b, **kw)
    check_forward(case, ref, out, "layernorm", "bf16", "f32", False, scaling, "e4m3", layout, scale)
    assert_ws_clean()


def test_element_aligned_tensors_backward():
    rows, hidden = 50, 2048
    case = workloads.small_case("layernorm", rows, hidden, "bf16", "f32", seed=13)
    ref_f = oracle_fwd(case, "layernorm", "bf16", "f32", False)
    ref = oracle_bwd(case, "layernorm", "bf16", "f32", False, ref_f)
    dy = offset_copy(case["dy"], 3)
    x = offset_copy(case["x"], 1)
    g = gpu(case, "gamma")[0]
    mu = torch.tensor(ref_f["mu"], dtype=torch.float32, device="cuda")
    rs = torch.tensor(ref_f["rsigma"], dtype=torch.float32, device="cuda")
    out = nf.bwd(dy, x, mu, rs, g, norm="layernorm")
    checks.check_dx(bits(out["dx"]), ref["dx"], "bf16")
    checks.check_wgrad(out["dgamma"].cpu().numpy(), ref["dgamma"])
    checks.check_wgrad(out["dbeta"].cpu().numpy(), ref["dbeta"], what="dbeta")


def test_general_zero_rows_delayed_colwise():
    """No rows: delayed scaling still publishes amax and both scale_inv values."""
    case = workloads.small_case("rmsnorm", 1, 100, "bf16", "f32", seed=1)
    x, g = gpu(case, "x", "gamma")
    am = torch.tensor([3.0], device="cuda")
    out = nf.fwd(x[:0], g, None, norm="rmsnorm", scaling="delayed", layout="colwise",
                 scale=torch.tensor([4.0], device="cuda"), amax=am)
    torch.cuda.synchronize()
    assert out["amax"].item() == 3.0 and out["colwise_scale_inv"].item() == 0.25
    assert_ws_clean()
