"""GPU parity on the method's degenerate and ill-conditioned inputs, against the oracle.

[XLA-Norm] "Implementation: NVIDIA TransformerEngine JAX XLA Normalization", I/O Contract: the
forward's epsilon input and its mu / rsigma outputs. Cases:
  * constant rows: biased variance 0, so rsigma = epsilon^-1/2 and LayerNorm gives y = beta;
  * all-zero RMSNorm rows: rsigma = epsilon^-1/2, y = 0; FP8 codes 0, amax 0, MXFP8 zero blocks
    (E8M0 byte 0);
  * large-mean LayerNorm rows (mean 1e3, standard deviation 1e-2 in float32; mean 100,
    deviation 1 in bf16), where a binary32 mean taken without care loses the deviations;
  * a delayed scale under which about a third of the elements saturate.
Every row layout class is covered by the hidden sizes (one wave, a team, a team with LDS
weights, the long-row layout, the band split, the general kernels).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import checks

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import rmsnorm_fp8_quantization_amd as nf  # noqa: E402

EPS = 1e-5
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}
HIDDEN = [1000, 1001, 1024, 4096, 8192, 12288, 65536, 98304]


def _case(norm, x, hidden, in_dt, seed):
    c = workloads.small_case(norm, x.shape[0], hidden, in_dt, "f32", seed=seed)
    c["x"] = x.to(TDT[in_dt])
    return c


def _fwd_check(case, norm, in_dt, **kw):
    bits = workloads.to_numpy_bits
    ref = oracle.forward_stored(bits(case["x"]), bits(case["gamma"]),
                                bits(case["beta"]) if norm == "layernorm" else None, norm=norm, eps=EPS,
                                in_dtype=in_dt, w_dtype="f32")
    x = case["x"].cuda()
    g = case["gamma"].cuda()
    b = case["beta"].cuda() if norm == "layernorm" else None
    out = nf.fwd(x, g, b, norm=norm, eps=EPS, **kw)
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None, out["rsigma"].cpu().numpy(),
                       ref["mu"], ref["rsigma"])
    return out, ref


def _ln_terms(case, ref):
    beta = oracle.decode_storage(workloads.to_numpy_bits(case["beta"]), "f32")[None, :]
    g = oracle.decode_storage(workloads.to_numpy_bits(case["gamma"]), "f32")[None, :]
    return np.abs(ref["v"] - beta) + np.abs(ref["mu"][:, None] * ref["rsigma"][:, None] * g) + np.abs(beta)


@pytest.mark.parametrize("hidden", HIDDEN)
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_constant_rows(norm, hidden):
    consts = torch.tensor([0.0, 3.5, -2.0, 1e-3, 250.0])
    x = consts[:, None].expand(len(consts), hidden).contiguous()
    case = _case(norm, x, hidden, "bf16", seed=hidden)
    out, ref = _fwd_check(case, norm, "bf16")
    print(f"constant rows {norm} hidden {hidden}", flush=True)
    # closed forms: LayerNorm rsigma = eps^-1/2 (to the hardware reciprocal square root's
    # accuracy), mu = the constant, y = beta (within the output tolerance)
    if norm == "layernorm":
        rs0 = 1.0 / np.sqrt(np.float64(np.float32(EPS)))
        assert np.all(np.abs(out["rsigma"].cpu().numpy() / rs0 - 1.0) <= 1e-6)
    checks.check_hp(workloads.to_numpy_bits(out["y"].cpu()), ref["v"], "bf16",
                    terms=_ln_terms(case, ref) if norm == "layernorm" else None)


@pytest.mark.parametrize("hidden", HIDDEN)
@pytest.mark.parametrize("scaling", ["none", "delayed", "mxfp8"])
def test_all_zero_rmsnorm_rows(hidden, scaling):
    rows = 64
    x = torch.zeros(rows, hidden)
    x[1::2] = torch.randn(rows // 2, hidden, generator=torch.Generator().manual_seed(hidden))
    case = _case("rmsnorm", x, hidden, "bf16", seed=hidden + 1)
    kw = {}
    if scaling == "delayed":
        kw = dict(scaling="delayed", fp8="e4m3", scale=torch.tensor([64.0], device="cuda"),
                  amax=torch.zeros(1, device="cuda"), layout="rowwise_colwise")
    elif scaling == "mxfp8":
        kw = dict(scaling="mxfp8", fp8="e4m3", layout="rowwise_colwise")
    print(f"zero rows {scaling} hidden {hidden}", flush=True)
    out, ref = _fwd_check(case, "rmsnorm", "bf16", **kw)
    rs = out["rsigma"].cpu().numpy()
    assert np.all(np.abs(rs[0::2] * np.sqrt(np.float64(np.float32(EPS))) - 1.0) <= 1e-6)
    y = workloads.to_numpy_bits(out["y"].cpu())
    assert np.all((y[0::2] & (0x7F if scaling != "none" else 0x7FFF)) == 0)   # zero codes / zero bf16
    if scaling == "none":
        checks.check_hp(y, ref["v"], "bf16")
    elif scaling == "delayed":
        got = {"y": y, "y_colwise": workloads.to_numpy_bits(out["y_colwise"].cpu()),
               "scale_inv": out["scale_inv"].item(), "colwise_scale_inv": out["colwise_scale_inv"].item(),
               "amax": out["amax"].item()}
        assert np.all((got["y_colwise"][:, 0::2] & 0x7F) == 0)
        checks.check_delayed(got, ref["v"], 64.0, 0.0, "e4m3", rowwise=True, colwise=True)
    else:
        s = workloads.to_numpy_bits(out["scale_inv"].cpu())
        assert np.all(s[0::2] == 0)                 # all-zero block: E8M0 byte 0
        checks.check_mx_rows(y, s, ref["v"], "e4m3", "mx rowwise")
        checks.check_mx_rows(workloads.to_numpy_bits(out["y_colwise"].cpu()),
                             workloads.to_numpy_bits(out["colwise_scale_inv"].cpu()),
                             np.ascontiguousarray(ref["v"].T), "e4m3", "mx colwise")


@pytest.mark.parametrize("hidden", HIDDEN)
@pytest.mark.parametrize("in_dt,mean,std", [("f32", 1e3, 1e-2), ("bf16", 100.0, 1.0)])
def test_large_mean_layernorm(hidden, in_dt, mean, std):
    rows = 24
    x = torch.randn(rows, hidden, generator=torch.Generator().manual_seed(hidden + 7), dtype=torch.float64)
    x = (x * std + mean).to(torch.float32)
    case = _case("layernorm", x, hidden, in_dt, seed=hidden + 2)
    print(f"large mean {in_dt} N({mean}, {std}) hidden {hidden}", flush=True)
    out, ref = _fwd_check(case, "layernorm", in_dt, out_dtype=TDT[in_dt])
    y = out["y"].cpu().numpy() if in_dt == "f32" else workloads.to_numpy_bits(out["y"].cpu())
    checks.check_hp(y, ref["v"], in_dt, terms=_ln_terms(case, ref) if in_dt != "f32" else None)


@pytest.mark.parametrize("hidden", [1024, 4096, 8192, 12288])
@pytest.mark.parametrize("fp8", ["e4m3", "e5m2"])
def test_delayed_scale_with_many_saturating_elements(hidden, fp8):
    """A scale four times the no-saturation scale: |y| * scale beyond the format's largest
    value for about a third of the elements; those codes must be the largest finite code."""
    rows = 96
    case = workloads.small_case("rmsnorm", rows, hidden, "bf16", "f32", seed=hidden + 3, x_mean=0.0, x_std=1.0)
    bits = workloads.to_numpy_bits
    ref = oracle.forward_stored(bits(case["x"]), bits(case["gamma"]), None, norm="rmsnorm", eps=EPS,
                                in_dtype="bf16", w_dtype="f32")
    fmax = 448.0 if fp8 == "e4m3" else 57344.0
    scale = float(np.float32(4.0 * fmax / np.max(np.abs(ref["v"]))))
    sat = np.abs(ref["v"] * scale) > fmax
    assert 0.002 < sat.mean() < 0.9, sat.mean()
    print(f"saturating delayed {fp8} hidden {hidden}: {sat.mean():.3f} of elements saturate", flush=True)
    out = nf.fwd(case["x"].cuda(), case["gamma"].cuda(), None, norm="rmsnorm", eps=EPS, scaling="delayed", fp8=fp8,
                 scale=torch.tensor([scale], device="cuda"), amax=torch.zeros(1, device="cuda"),
                 layout="rowwise_colwise")
    got = {"y": bits(out["y"].cpu()), "y_colwise": bits(out["y_colwise"].cpu()), "scale_inv": out["scale_inv"].item(),
           "colwise_scale_inv": out["colwise_scale_inv"].item(), "amax": out["amax"].item()}
    checks.check_delayed(got, ref["v"], scale, 0.0, fp8, rowwise=True, colwise=True)
    maxcode = 0x7E if fp8 == "e4m3" else 0x7B
    assert np.all((got["y"][sat] & 0x7F) == maxcode)
