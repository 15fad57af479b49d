"""GPU: calls captured in a HIP graph replay to the same results as eager calls, and to the
oracle's.

The library enqueues only kernels (no memset or copy nodes) on the caller's stream, and its
workspace header carries a launch epoch in device memory, so a captured forward / backward can
be replayed: every replay, with new inputs copied into the captured buffers and eager work and
synchronisation in between, must match an eager call on the same inputs bit for bit. Covered:
the LayerNorm forward + backward, the delayed-scaling columnwise forward (cross-workgroup amax
through the workspace), and the MXFP8 columnwise forward. Every replay is also checked against
the oracle, and one test makes a larger call on the capture stream between capture and replay
(the binding's workspace for that stream grows; the captured calls keep theirs).
[XLA-Norm] "Implementation: NVIDIA TransformerEngine JAX XLA Normalization", Description: the
"Initialize" variants of the forward and backward, for graph capture.
"""
import numpy as np
import pytest
import torch

import checks
import workloads
from test_gpu_parity import bits, ln_terms, oracle_bwd, oracle_fwd

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import rmsnorm_fp8_quantization_amd as nf  # noqa: E402

EPS = 1e-5


def _kw(mode):
    if mode == "delayed":
        return dict(norm="rmsnorm", scaling="delayed", fp8="e4m3", layout="rowwise_colwise",
                    scale=torch.tensor([12.0], device="cuda"), amax=torch.zeros(1, device="cuda"))
    if mode == "mxfp8":
        return dict(norm="rmsnorm", scaling="mxfp8", fp8="e4m3", layout="rowwise_colwise")
    return dict(norm="layernorm")


@pytest.mark.parametrize("mode", ["plain", "delayed", "mxfp8"])
def test_graph_replay_matches_eager(mode):
    rows, hidden = 640, 1536
    norm = "layernorm" if mode == "plain" else "rmsnorm"
    cases = [workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=50 + i) for i in range(3)]
    g = cases[0]["gamma"].cuda()
    b = cases[0]["beta"].cuda() if norm == "layernorm" else None
    kw = _kw(mode)
    x_static = cases[0]["x"].cuda()
    dy_static = cases[0]["dy"].cuda()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):  # warm-up on the capture stream: its workspace is allocated here
            f = nf.fwd(x_static, g, b, **kw)
            if mode == "plain":
                nf.bwd(dy_static, x_static, f["mu"], f["rsigma"], g, norm=norm)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        fo = nf.fwd(x_static, g, b, **kw)
        bo = nf.bwd(dy_static, x_static, fo["mu"], fo["rsigma"], g, norm=norm) if mode == "plain" else {}

    for i, c in enumerate(cases * 2):
        x_static.copy_(c["x"].cuda())
        dy_static.copy_(c["dy"].cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in {**fo, **bo}.items() if v is not None}
        # eager reference on the same inputs (its own buffers; the default stream's workspace)
        ef = nf.fwd(x_static.clone(), g, b, **kw)
        eb = nf.bwd(dy_static.clone(), x_static.clone(), ef["mu"], ef["rsigma"], g, norm=norm) \
            if mode == "plain" else {}
        torch.cuda.synchronize()
        for k, v in {**ef, **eb}.items():
            if v is None:
                continue
            assert torch.equal(got[k], v), f"replay {i}: {k} differs from the eager call"
        # (the captured calls read the weights of cases[0]; x and dy are this case's)
        check_against_oracle({**c, "gamma": cases[0]["gamma"], "beta": cases[0].get("beta")}, mode, got, kw)


def check_against_oracle(c, mode, got, kw):
    norm = "layernorm" if mode == "plain" else "rmsnorm"
    ref = oracle_fwd(c, norm, "bf16", "f32", False)
    checks.check_stats(None if got.get("mu") is None else got["mu"].cpu().numpy(), got["rsigma"].cpu().numpy(),
                       ref["mu"], ref["rsigma"])
    if mode == "plain":
        checks.check_hp(bits(got["y"]), ref["v"], "bf16", terms=ln_terms(c, ref, norm))
        rb = oracle_bwd(c, norm, "bf16", "f32", False, ref)
        checks.check_dx(bits(got["dx"]), rb["dx"], "bf16")
        checks.check_wgrad(got["dgamma"].cpu().numpy(), rb["dgamma"])
        checks.check_wgrad(got["dbeta"].cpu().numpy(), rb["dbeta"], what="dbeta")
    elif mode == "delayed":
        out = {"y": bits(got["y"]), "y_colwise": bits(got["y_colwise"]), "scale_inv": got["scale_inv"].item(),
               "colwise_scale_inv": got["colwise_scale_inv"].item(), "amax": got["amax"].item()}
        checks.check_delayed(out, ref["v"], kw["scale"].item(), 0.0, "e4m3", rowwise=True, colwise=True)
    else:
        checks.check_mx_rows(bits(got["y"]), bits(got["scale_inv"]), ref["v"], "e4m3", "mx rowwise")
        checks.check_mx_rows(bits(got["y_colwise"]), bits(got["colwise_scale_inv"]),
                             np.ascontiguousarray(ref["v"].T), "e4m3", "mx colwise")


@pytest.mark.parametrize("mode", ["plain", "delayed"])
def test_graph_replay_after_a_larger_call_on_the_capture_stream(mode):
    """A call on the capture stream that needs a larger workspace than the captured calls makes
    the binding replace that stream's cached workspace; the captured calls still point at the
    old one, which must stay allocated: replays after it match the oracle."""
    rows, hidden = 512, 2048
    norm = "layernorm" if mode == "plain" else "rmsnorm"
    c = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=71)
    g = c["gamma"].cuda()
    b = c["beta"].cuda() if norm == "layernorm" else None
    kw = _kw(mode)
    x_static = c["x"].cuda()
    dy_static = c["dy"].cuda()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        f = nf.fwd(x_static, g, b, **kw)  # warm-up: this stream's workspace is allocated here
        if mode == "plain":
            nf.bwd(dy_static, x_static, f["mu"], f["rsigma"], g, norm=norm)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        fo = nf.fwd(x_static, g, b, **kw)
        bo = nf.bwd(dy_static, x_static, fo["mu"], fo["rsigma"], g, norm=norm) if mode == "plain" else {}
    # a much larger call on the capture stream: its workspace need exceeds the cached one
    big = workloads.small_case(norm, 8192, 8192, "bf16", "f32", seed=72)
    with torch.cuda.stream(s):
        bx, bdy = big["x"].cuda(), big["dy"].cuda()
        bg = big["gamma"].cuda()
        bb = big["beta"].cuda() if norm == "layernorm" else None
        bf = nf.fwd(bx, bg, bb, **kw)
        if mode == "plain":
            nf.bwd(bdy, bx, bf["mu"], bf["rsigma"], bg, norm=norm)
    torch.cuda.synchronize()
    del bx, bdy, bf
    torch.cuda.empty_cache()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in {**fo, **bo}.items() if v is not None}
        check_against_oracle(c, mode, got, kw)
