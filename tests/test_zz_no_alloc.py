"""GPU test of norm_bwd_noalloc (the backward whose scratch memory is a static device array)
against norm_bwd with a caller workspace, and against the oracle.

Two calls in a row, the second with a smaller input, so the second call runs on a scratch array
that still holds the first call's partials. Called through the C ABI with explicit pointers.
[NVRTC-PR] "Migrate norms and softmax kernels to NVRTC", Flowchart (partial kernels, finalize).
"""
import ctypes

import pytest
import torch

import oracle
import workloads
import checks

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from rmsnorm_fp8_quantization_amd import _lib as L, ops  # noqa: E402

EPS = 1e-5
NORM = {"layernorm": L.NORM_LAYERNORM, "rmsnorm": L.NORM_RMSNORM}


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _inputs(norm, rows, hidden, seed):
    case = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=seed)
    bits = workloads.to_numpy_bits
    ref_f = oracle.forward_stored(bits(case["x"]), bits(case["gamma"]),
                                  bits(case["beta"]) if norm == "layernorm" else None, norm=norm, eps=EPS,
                                  in_dtype="bf16", w_dtype="f32")
    ref = oracle.backward_stored(bits(case["dy"]), bits(case["x"]), ref_f["mu"], ref_f["rsigma"], bits(case["gamma"]),
                                 norm=norm, in_dtype="bf16", w_dtype="f32")
    dev = torch.device("cuda")
    t = {k: case[k].to(dev) for k in ("dy", "x", "gamma")}
    t["mu"] = torch.tensor(ref_f["mu"], dtype=torch.float32, device=dev) if norm == "layernorm" else None
    t["rs"] = torch.tensor(ref_f["rsigma"], dtype=torch.float32, device=dev)
    return t, ref


def _outputs(t, norm):
    dx = torch.empty_like(t["x"])
    dg = torch.empty_like(t["gamma"])
    db = torch.empty_like(t["gamma"]) if norm == "layernorm" else None
    return dx, dg, db


def _noalloc(t, norm, rows, hidden):
    dx, dg, db = _outputs(t, norm)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L.call("norm_bwd_noalloc", stream, _p(t["dy"]), _p(t["x"]), _p(t["mu"]), _p(t["rs"]), _p(t["gamma"]), _p(dx),
           _p(dg), _p(db), rows, hidden, L.NORM_BF16, L.NORM_F32, NORM[norm], 0, 0)
    return dx, dg, db


def _with_workspace(t, norm, rows, hidden):
    dx, dg, db = _outputs(t, norm)
    nbytes = ops.bwd_workspace_size(rows, hidden, torch.bfloat16, torch.float32, norm)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L.call("norm_bwd", stream, _p(t["dy"]), _p(t["x"]), _p(t["mu"]), _p(t["rs"]), _p(t["gamma"]), _p(dx), _p(dg),
           _p(db), _p(ws), ws.numel(), rows, hidden, L.NORM_BF16, L.NORM_F32, NORM[norm], 0, 0)
    return dx, dg, db


@pytest.mark.parametrize("norm,first,second", [
    ("layernorm", (16384, 4096), (3000, 1024)),
    ("rmsnorm", (8192, 8192), (777, 2048)),
])
def test_noalloc_matches_workspace_backward_twice(norm, first, second):
    for rows, hidden in (first, second):
        print(f"noalloc {norm} {rows}x{hidden}", flush=True)
        t, ref = _inputs(norm, rows, hidden, seed=rows + hidden)
        got = _noalloc(t, norm, rows, hidden)
        want = _with_workspace(t, norm, rows, hidden)
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            if a is not None:
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))   # same kernels, same plan
        checks.check_dx(workloads.to_numpy_bits(got[0].cpu()), ref["dx"], "bf16")
        checks.check_wgrad(got[1].cpu().numpy(), ref["dgamma"])
        if got[2] is not None:
            checks.check_wgrad(got[2].cpu().numpy(), ref["dbeta"], what="dbeta")


def test_noalloc_rejects_shapes_beyond_the_scratch_array():
    t, _ = _inputs("layernorm", 4, 64, seed=1)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dx = torch.empty(1, dtype=torch.bfloat16, device="cuda")
    rc = L.status("norm_bwd_noalloc", stream, _p(t["dy"]), _p(t["x"]), _p(t["mu"]), _p(t["rs"]), _p(t["gamma"]),
                  _p(dx), _p(dx), _p(dx), 4, 1 << 20, L.NORM_BF16, L.NORM_F32, L.NORM_LAYERNORM, 0, 0)
    assert rc == L.NORM_ERR_UNSUPPORTED
    assert b"static buffer" in L.load().norm_last_error()
