"""GPU: the torch.autograd functions route to the same kernels as the direct calls, and their
results match the oracle.

Each check is bit-exact against the direct ``fwd`` / ``bwd`` / ``bwd_add`` calls on the same
inputs, then against the oracle (y from the oracle's forward; dx, dgamma, dbeta from its
backward at its own statistics, the end-to-end check of the GPU forward feeding the GPU
backward), plus a loose comparison with torch's own float32 autograd of the same formula as a
plumbing check (shapes, which gradient goes where, zero-centred gamma, the residual branch).
[BwdAdd] "Implementation: NVIDIA TransformerEngine Ops Fused Backward Add RMSNorm", Usage and
I/O Contract: the fused backward-add pattern (the residual branch's gradient added into dx).
"""
import pytest
import torch

import checks
import workloads
from test_gpu_parity import bits, ln_terms, oracle_bwd, oracle_fwd

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import rmsnorm_fp8_quantization_amd as nf  # noqa: E402
from rmsnorm_fp8_quantization_amd import autograd as A  # noqa: E402

EPS = 1e-5
SHAPE = (3, 40, 776)  # leading dims flattened to 120 rows; 776 = 97 strips (ragged)


def torch_ref(x, g, b, norm, zc):
    """float32 torch formula (autograd reference)."""
    xf = x.float()
    w = g.float() + 1.0 if zc else g.float()
    if norm == "layernorm":
        mu = xf.mean(-1, keepdim=True)
        var = ((xf - mu) ** 2).mean(-1, keepdim=True)
        return (xf - mu) * torch.rsqrt(var + EPS) * w + b.float()
    return xf * torch.rsqrt((xf * xf).mean(-1, keepdim=True) + EPS) * w


@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("zc", [False, True])
def test_autograd_norm(norm, zc):
    rows, hidden = SHAPE[0] * SHAPE[1], SHAPE[2]
    c = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=31, zero_centered_gamma=zc)
    x = c["x"].cuda().view(SHAPE).requires_grad_()
    g = c["gamma"].cuda().requires_grad_()
    b = c["beta"].cuda().requires_grad_() if norm == "layernorm" else None
    dy = c["dy"].cuda().view(SHAPE)
    y = A.layer_norm(x, g, b, EPS, zc) if norm == "layernorm" else A.rms_norm(x, g, EPS, zc)
    assert y.shape == SHAPE and y.dtype == torch.bfloat16
    y.backward(dy)

    x2 = x.detach().view(rows, hidden)
    f = nf.fwd(x2, g.detach(), None if b is None else b.detach(), norm=norm, eps=EPS,
               zero_centered_gamma=zc)
    d = nf.bwd(dy.view(rows, hidden), x2, f["mu"], f["rsigma"], g.detach(), norm=norm,
               zero_centered_gamma=zc)
    assert torch.equal(y.detach().view(rows, hidden), f["y"])
    assert torch.equal(x.grad.view(rows, hidden), d["dx"])
    assert torch.equal(g.grad, d["dgamma"])
    if b is not None:
        assert torch.equal(b.grad, d["dbeta"])

    # against the oracle: forward values and statistics, then the backward end to end
    ref_f = oracle_fwd(c, norm, "bf16", "f32", zc)
    checks.check_stats(None if f["mu"] is None else f["mu"].cpu().numpy(), f["rsigma"].cpu().numpy(),
                       ref_f["mu"], ref_f["rsigma"])
    checks.check_hp(bits(y.detach().view(rows, hidden)), ref_f["v"], "bf16", terms=ln_terms(c, ref_f, norm, zc=zc))
    ref_b = oracle_bwd(c, norm, "bf16", "f32", zc, ref_f)
    checks.check_dx(bits(x.grad.view(rows, hidden)), ref_b["dx"], "bf16")
    checks.check_wgrad(g.grad.cpu().numpy(), ref_b["dgamma"])
    if b is not None:
        checks.check_wgrad(b.grad.cpu().numpy(), ref_b["dbeta"], what="dbeta")

    # plumbing against torch's float32 autograd (bf16 rounding of y and dx bounds the difference)
    xr = x.detach().clone().requires_grad_()
    gr = g.detach().clone().requires_grad_()
    br = None if b is None else b.detach().clone().requires_grad_()
    yr = torch_ref(xr, gr, br, norm, zc)
    yr.backward(dy.float())
    torch.testing.assert_close(y.float(), yr, atol=0.05, rtol=0.02)
    torch.testing.assert_close(x.grad.float(), xr.grad.float(), atol=0.05, rtol=0.05)
    torch.testing.assert_close(g.grad, gr.grad, atol=0.5, rtol=0.02)
    if b is not None:
        torch.testing.assert_close(b.grad, br.grad, atol=0.05, rtol=0.01)


@pytest.mark.parametrize("zc", [False, True])
def test_autograd_rms_norm_residual(zc):
    rows, hidden = SHAPE[0] * SHAPE[1], SHAPE[2]
    c = workloads.small_case("rmsnorm", rows, hidden, "bf16", "f32", seed=37, zero_centered_gamma=zc)
    x = c["x"].cuda().view(SHAPE).requires_grad_()
    g = c["gamma"].cuda().requires_grad_()
    dy = c["dy"].cuda().view(SHAPE)
    dres = c["residual_dy"].cuda().view(SHAPE)
    y, xres = A.rms_norm_residual(x, g, EPS, zc)
    assert xres.data_ptr() == x.data_ptr()          # the residual branch gets x itself
    torch.autograd.backward([y, xres], [dy, dres])

    x2 = x.detach().view(rows, hidden)
    f = nf.fwd(x2, g.detach(), None, norm="rmsnorm", eps=EPS, zero_centered_gamma=zc)
    d = nf.bwd_add(dy.view(rows, hidden), x2, dres.view(rows, hidden), f["rsigma"], g.detach(),
                   zero_centered_gamma=zc)
    assert torch.equal(y.detach().view(rows, hidden), f["y"])
    assert torch.equal(x.grad.view(rows, hidden), d["dx"])
    assert torch.equal(g.grad, d["dgamma"])

    # against the oracle: dx = RMSNorm backward + residual gradient, and dgamma
    ref_f = oracle_fwd(c, "rmsnorm", "bf16", "f32", zc)
    checks.check_hp(bits(y.detach().view(rows, hidden)), ref_f["v"], "bf16")
    ref_b = oracle_bwd(c, "rmsnorm", "bf16", "f32", zc, ref_f, add=True)
    checks.check_dx(bits(x.grad.view(rows, hidden)), ref_b["dx"], "bf16")
    checks.check_wgrad(g.grad.cpu().numpy(), ref_b["dgamma"])

    # only the norm output used: the plain backward, no residual term
    x.grad = None
    g.grad = None
    y, xres = A.rms_norm_residual(x, g, EPS, zc)
    y.backward(dy)
    d0 = nf.bwd(dy.view(rows, hidden), x2, None, f["rsigma"], g.detach(), norm="rmsnorm",
                zero_centered_gamma=zc)
    assert torch.equal(x.grad.view(rows, hidden), d0["dx"])
    assert torch.equal(g.grad, d0["dgamma"])
