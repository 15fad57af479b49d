"""GPU: calls captured in a HIP graph replay to the same results as eager calls.

The library enqueues only kernels (no memset or copy nodes) on the caller's stream, and its
workspace header carries a launch epoch in device memory, so a captured forward / backward can
be replayed: every replay, with new inputs copied into the captured buffers and eager work and
synchronisation in between, must match an eager call on the same inputs bit for bit. Covered:
the LayerNorm forward + backward, the delayed-scaling columnwise forward (cross-workgroup amax
through the workspace), and the MXFP8 columnwise forward.
"""
import pytest
import torch

import workloads

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
