"""GPU parity: the HIP library (called through its C ABI via the binding) against the CPU oracle.

Inputs are seeded synthetic tensors from ``workloads``; the same host arrays feed both sides.
Shapes span several tiles and ragged tails; every forward layout (wave / workgroup team,
band split, columnwise band) is forced on small shapes through the planner's override knobs.
Tolerances are those of tests/checks.py.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import formats as F
import checks

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import rmsnorm_fp8_quantization_amd as nf  # noqa: E402

TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
EPS = 1e-5


def env(**kv):
    """Planner overrides for a block (norm_tuning_set through the binding)."""
    return nf._lib.tuning(**kv)


def bits(t):
    return workloads.to_numpy_bits(t.cpu())


def host_np(t, dtype):
    """Stored values of a host tensor as the oracle's storage arrays."""
    return workloads.to_numpy_bits(t)


def oracle_fwd(case, norm, in_dt, w_dt, zc):
    return oracle.forward_stored(host_np(case["x"], in_dt), host_np(case["gamma"], w_dt),
                                 host_np(case["beta"], w_dt) if norm == "layernorm" else None,
                                 norm=norm, eps=EPS, in_dtype=in_dt, w_dtype=w_dt, zero_centered_gamma=zc)


def ln_terms(case, ref, norm, w_dt="f32", zc=False):
    """|xhat * g| + |mu * rsigma * g| + |beta| per element (LayerNorm): the magnitude of the
    terms whose binary32 sum gives y (x * rsigma * g, the mean's share, beta)."""
    if norm != "layernorm":
        return None
    beta = F.decode_storage(host_np(case["beta"], w_dt), w_dt)[None, :]
    g = oracle.effective_gamma(F.decode_storage(host_np(case["gamma"], w_dt), w_dt), zc)[None, :]
    mu_share = np.abs(ref["mu"][:, None] * ref["rsigma"][:, None] * g)
    return np.abs(ref["v"] - beta) + mu_share + np.abs(beta)


def T(a):
    """Transpose of a per-element array (None stays None)."""
    return None if a is None else np.ascontiguousarray(a.T)


def gpu(case, *names):
    return [case[n].cuda() if n in case else None for n in names]


def assert_ws_clean():
    torch.cuda.synchronize()
    assert nf.workspace_check() == 0


# ------------------------------------------------------------------------------ plain forward

PLAIN_SHAPES = [(1, 8), (3, 200), (37, 1024), (64, 4096), (5, 4104), (7, 8192), (3, 16384), (2, 20480),
                (4, 65536), (300, 512)]


@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("in_dt", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("rows,hidden", PLAIN_SHAPES)
def test_fwd_plain(norm, in_dt, rows, hidden):
    case = workloads.small_case(norm, rows, hidden, in_dt, "f32", seed=rows + hidden)
    ref = oracle_fwd(case, norm, in_dt, "f32", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    out = nf.fwd(x, g, b, norm=norm, eps=EPS)
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                       out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    checks.check_hp(bits(out["y"]), ref["v"], in_dt, terms=ln_terms(case, ref, norm))


@pytest.mark.parametrize("out_dt", ["f32", "f16"])
def test_fwd_plain_other_out_dtype_and_bf16_weights(out_dt):
    case = workloads.small_case("layernorm", 33, 3000 - 3000 % 8, "bf16", "bf16", seed=3)
    ref = oracle_fwd(case, "layernorm", "bf16", "bf16", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    out = nf.fwd(x, g, b, norm="layernorm", eps=EPS, out_dtype=TDT[out_dt])
    checks.check_hp(bits(out["y"]), ref["v"], out_dt, terms=ln_terms(case, ref, "layernorm", "bf16"))


ROW_COVER = [512, 1024, 2048, 4096, 4096, 8192, 16384, 4096, 4096, 4096, 65536, 8192, 16384, 16384,
             32768, 32768, 16384]   # per row layout
BWD_COVER = [1024, 2048, 4096, 8192, 16384, 4096, 8192, 8192, 1024, 2048, 4096, 12288, 5120, 5120]


@pytest.mark.parametrize("cfg", range(len(ROW_COVER)))
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_fwd_every_row_layout(cfg, norm):
    hidden = ROW_COVER[cfg] - 8   # ragged: the last strip of the row is masked
    rows = 19
    case = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=cfg)
    ref = oracle_fwd(case, norm, "bf16", "f32", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    with env(NORMFP8_ROW_CFG=cfg):
        out = nf.fwd(x, g, b, norm=norm, eps=EPS)
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                       out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    checks.check_hp(bits(out["y"]), ref["v"], "bf16", terms=ln_terms(case, ref, norm))


@pytest.mark.parametrize("in_dt,out_dt", [("f16", "f16"), ("bf16", "f32"), ("f16", "bf16")])
@pytest.mark.parametrize("rows,hidden", [(7, 16392), (37, 24576), (3, 32768), (600, 16400), (5, 8200),
                                         (1100, 12288), (9, 16384)])
def test_fwd_layernorm_8k_to_32k_register_weights(in_dt, out_dt, rows, hidden):
    """LayerNorm rows of 8193..32768 elements with a 16-bit input and no FP8 epilogue: 4 waves
    (8193..16384) or 8 waves (16385..32768) per row with gamma and beta in registers for the
    whole persistent workgroup and the next row prefetched (600 and 1100 rows: several rows per
    workgroup, a ragged last round)."""
    case = workloads.small_case("layernorm", rows, hidden, in_dt, "f32", seed=rows + hidden)
    ref = oracle_fwd(case, "layernorm", in_dt, "f32", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    print(f"ln 8k-32k: {rows}x{hidden} {in_dt}->{out_dt}", flush=True)
    out = nf.fwd(x, g, b, norm="layernorm", eps=EPS, out_dtype=TDT[out_dt])
    checks.check_hp(bits(out["y"]), ref["v"], out_dt, terms=ln_terms(case, ref, "layernorm"))
    checks.check_stats(out["mu"].cpu().numpy(), out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    assert_ws_clean()


# rows of 32769..65536 elements: 16 waves x 8 strips, weights read from the caches a strip ahead
# of their use; rows of 16385..32768: 16 waves x 4 strips (RMSNorm's gamma in registers,
# LayerNorm's gamma and beta from the caches); rows of 8193..16384 elements: RMSNorm FP8 epilogues on 8 waves x
# 4 strips, its plain outputs on 16 waves x 2 strips, LayerNorm on two 8-wave rows per
# workgroup sharing the LDS weights; RMSNorm FP8 rowwise epilogues at 2049..4096 elements on
# 4 waves x 2 rows x 2 strips (any weight dtype, zero-centred gamma, every rowwise epilogue)
@pytest.mark.parametrize("w_dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("mode", ["none", "delayed", "mxfp8"])
@pytest.mark.parametrize("norm,hidden,zc", [("layernorm", 65536, False), ("rmsnorm", 65536, True),
                                            ("layernorm", 40000, True), ("rmsnorm", 20488, False),
                                            ("layernorm", 32768, False), ("rmsnorm", 32760, True),
                                            ("layernorm", 16392, True),
                                            ("rmsnorm", 12288, True), ("rmsnorm", 10232, False),
                                            ("rmsnorm", 16384, False), ("layernorm", 12288, True),
                                            ("layernorm", 10232, False), ("rmsnorm", 4096, True),
                                            ("rmsnorm", 2056, False), ("layernorm", 45056, False),
                                            ("rmsnorm", 98304, False), ("rmsnorm", 196608, True)])
def test_fwd_long_rows(w_dt, mode, norm, hidden, zc):
    rows = 5
    case = workloads.small_case(norm, rows, hidden, "bf16", w_dt, seed=hidden % 97 + rows, zero_centered_gamma=zc)
    ref = oracle_fwd(case, norm, "bf16", w_dt, zc)
    x, g, b = gpu(case, "x", "gamma", "beta")
    t = ln_terms(case, ref, norm, w_dt, zc)
    if mode == "none":
        out = nf.fwd(x, g, b, norm=norm, eps=EPS, zero_centered_gamma=zc)
        checks.check_hp(bits(out["y"]), ref["v"], "bf16", terms=t)
    elif mode == "delayed":
        scale = float(np.float32(F.E4M3.max_finite) / np.float32(np.max(np.abs(ref["v"]))))
        st = torch.tensor([scale], dtype=torch.float32, device="cuda")
        am = torch.zeros(1, dtype=torch.float32, device="cuda")
        out = nf.fwd(x, g, b, norm=norm, eps=EPS, zero_centered_gamma=zc, scaling="delayed", fp8="e4m3",
                     scale=st, amax=am, layout="rowwise")
        got = {"y": bits(out["y"]), "y_colwise": None, "scale_inv": out["scale_inv"].item(),
               "colwise_scale_inv": None, "amax": out["amax"].item()}
        checks.check_delayed(got, ref["v"], scale, 0.0, "e4m3", rowwise=True, colwise=False, terms=t)
    else:
        out = nf.fwd(x, g, b, norm=norm, eps=EPS, zero_centered_gamma=zc, scaling="mxfp8", fp8="e4m3",
                     layout="rowwise")
        checks.check_mx_rows(bits(out["y"]), bits(out["scale_inv"]), ref["v"], "e4m3", "mx rowwise", terms=t)
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                       out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    assert_ws_clean()


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("rows,hidden", [(37, 1000), (9, 12288)])
def test_fwd_forced_band_split(cfg, norm, rows, hidden):
    case = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=cfg + 50)
    ref = oracle_fwd(case, norm, "bf16", "f32", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    with env(NORMFP8_FORCE_BAND=1, NORMFP8_BAND_CFG=cfg):
        out = nf.fwd(x, g, b, norm=norm, eps=EPS)
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                       out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    checks.check_hp(bits(out["y"]), ref["v"], "bf16", terms=ln_terms(case, ref, norm))
    assert_ws_clean()


def test_fwd_zero_centered_gamma_and_zero_rows():
    case = workloads.small_case("rmsnorm", 11, 768, "bf16", "f32", seed=9, zero_centered_gamma=True)
    ref = oracle_fwd(case, "rmsnorm", "bf16", "f32", True)
    x, g = gpu(case, "x", "gamma")
    out = nf.fwd(x, g, None, norm="rmsnorm", eps=EPS, zero_centered_gamma=True)
    checks.check_hp(bits(out["y"]), ref["v"], "bf16")
    empty = nf.fwd(x[:0], g, None, norm="rmsnorm", eps=EPS)
    assert empty["y"].shape == (0, 768)


# ------------------------------------------------------------------------------ delayed scaling

@pytest.mark.parametrize("fp8", ["e4m3", "e5m2"])
@pytest.mark.parametrize("layout", ["rowwise", "rowwise_colwise", "colwise"])
@pytest.mark.parametrize("norm,rows,hidden", [("rmsnorm", 64, 1024), ("rmsnorm", 45, 4104),
                                              ("layernorm", 100, 2048), ("rmsnorm", 33, 20480),
                                              ("layernorm", 50, 4096), ("rmsnorm", 130, 3072),
                                              ("layernorm", 40, 5120), ("layernorm", 24, 10240)])
def test_fwd_delayed(fp8, layout, norm, rows, hidden):
    case = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=rows)
    xh = case["x"].float()
    xh[::7, ::13] *= 20.0                       # outliers beyond the scale's range
    case["x"] = xh.to(torch.bfloat16)
    ref = oracle_fwd(case, norm, "bf16", "f32", False)
    scale = float(np.float32(F.E4M3.max_finite if fp8 == "e4m3" else F.E5M2.max_finite) /
                  np.float32(np.max(np.abs(ref["v"])) / 4))
    x, g, b = gpu(case, "x", "gamma", "beta")
    st = torch.tensor([scale], dtype=torch.float32, device="cuda")
    am = torch.tensor([0.25], dtype=torch.float32, device="cuda")
    out = nf.fwd(x, g, b, norm=norm, eps=EPS, scaling="delayed", fp8=fp8, scale=st, amax=am, layout=layout)
    got = {"y": bits(out["y"]) if out["y"] is not None else None,
           "y_colwise": bits(out["y_colwise"]) if out["y_colwise"] is not None else None,
           "scale_inv": out["scale_inv"].item() if out["scale_inv"] is not None else None,
           "colwise_scale_inv": out["colwise_scale_inv"].item() if out["colwise_scale_inv"] is not None else None,
           "amax": out["amax"].item()}
    checks.check_delayed(got, ref["v"], scale, 0.25, fp8, rowwise=layout != "colwise",
                         colwise=layout != "rowwise", terms=ln_terms(case, ref, norm))
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                       out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    assert_ws_clean()


@pytest.mark.parametrize("rl,tc", [("8", "256"), ("4", "256"), ("8", "128")])
@pytest.mark.parametrize("rows,hidden", [(300, 4096), (129, 8192), (37, 2064), (256, 512), (1, 16), (512, 768),
                                         (1100, 400), (64, 12288)])
def test_fwd_delayed_transpose_path_matches_tiles(rows, hidden, rl, tc):
    """Delayed scaling with both outputs: the row kernel + byte transpose path (each tile
    shape: 256 or 128 rows x 256 columns, 512 rows x 128 columns) gives the same bytes as the
    statistics + tile path, and both match the oracle."""
    case = workloads.small_case("rmsnorm", rows, hidden, "bf16", "f32", seed=rows + 11)
    xh = case["x"].float()
    xh[::5, ::11] *= 20.0
    case["x"] = xh.to(torch.bfloat16)
    ref = oracle_fwd(case, "rmsnorm", "bf16", "f32", False)
    scale = float(np.float32(448.0) / np.float32(np.max(np.abs(ref["v"])) / 2))
    x, g = gpu(case, "x", "gamma")
    outs = []
    for knob in ("1", "0"):
        with env(NORMFP8_DELAYED_TRANSPOSE=knob, NORMFP8_TRANSPOSE_RL=rl, NORMFP8_TRANSPOSE_TC=tc):
            o = nf.fwd(x, g, None, norm="rmsnorm", eps=EPS, scaling="delayed", fp8="e4m3", layout="rowwise_colwise",
                       scale=torch.tensor([scale], device="cuda"), amax=torch.zeros(1, device="cuda"))
        torch.cuda.synchronize()
        outs.append(o)
        got = {"y": bits(o["y"]), "y_colwise": bits(o["y_colwise"]), "scale_inv": o["scale_inv"].item(),
               "colwise_scale_inv": o["colwise_scale_inv"].item(), "amax": o["amax"].item()}
        checks.check_delayed(got, ref["v"], scale, 0.0, "e4m3", rowwise=True, colwise=True)
    a, b = outs
    for k in ("y", "y_colwise", "rsigma", "scale_inv", "colwise_scale_inv", "amax"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["y_colwise"], a["y"].t().contiguous())
    assert_ws_clean()


def test_fwd_delayed_amax_inplace_and_accumulates():
    case = workloads.small_case("rmsnorm", 16, 512, "bf16", "f32", seed=2)
    ref = oracle_fwd(case, "rmsnorm", "bf16", "f32", False)
    x, g = gpu(case, "x", "gamma")
    st = torch.tensor([100.0], device="cuda")
    am = torch.tensor([1e4], device="cuda")          # larger than max |y|: kept
    out = nf.fwd(x, g, None, norm="rmsnorm", scaling="delayed", scale=st, amax=am, amax_inplace=True)
    torch.cuda.synchronize()
    assert out["amax"].data_ptr() == am.data_ptr() and am.item() == 1e4
    am.zero_()
    nf.fwd(x, g, None, norm="rmsnorm", scaling="delayed", scale=st, amax=am, amax_inplace=True)
    assert abs(am.item() - np.max(np.abs(ref["v"]))) <= 1e-6 * np.max(np.abs(ref["v"]))
    assert_ws_clean()


# ------------------------------------------------------------------------------ MXFP8

@pytest.mark.parametrize("fp8", ["e4m3", "e5m2"])
@pytest.mark.parametrize("layout", ["rowwise", "rowwise_colwise", "colwise"])
@pytest.mark.parametrize("norm,rows,hidden,zc", [("rmsnorm", 64, 1024, True), ("rmsnorm", 45, 1000, False),
                                                 ("layernorm", 96, 4096, False), ("rmsnorm", 32, 12288, True),
                                                 ("rmsnorm", 7, 512, False), ("layernorm", 40, 6144, False),
                                                 ("layernorm", 24, 10240, True)])
def test_fwd_mxfp8(fp8, layout, norm, rows, hidden, zc):
    case = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=hidden + rows, zero_centered_gamma=zc)
    ref = oracle_fwd(case, norm, "bf16", "f32", zc)
    x, g, b = gpu(case, "x", "gamma", "beta")
    out = nf.fwd(x, g, b, norm=norm, eps=EPS, zero_centered_gamma=zc, scaling="mxfp8", fp8=fp8, layout=layout)
    t = ln_terms(case, ref, norm, zc=zc)
    if layout != "colwise":
        checks.check_mx_rows(bits(out["y"]), bits(out["scale_inv"]), ref["v"], fp8, "mx rowwise", terms=t)
    if layout != "rowwise":
        checks.check_mx_rows(bits(out["y_colwise"]), bits(out["colwise_scale_inv"]),
                             np.ascontiguousarray(ref["v"].T), fp8, "mx colwise", terms=T(t))
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                       out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    assert_ws_clean()


# padded E8M0 grids (block-count dimension to a multiple of 4, the other to 128): the same codes
# and logical scales as the unpadded layout, the padding left as the caller filled it
SENTINEL = 0xA5


def _padded_case(path, layout, norm, rows, hidden):
    case = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=rows + hidden + 3)
    x, g, b = gpu(case, "x", "gamma", "beta")
    knobs = {"band": dict(NORMFP8_FORCE_BAND=1, NORMFP8_COL_KERNEL=0)}.get(path, {})
    kw = dict(norm=norm, eps=EPS, scaling="mxfp8", fp8="e4m3", layout=layout)
    with env(**knobs):
        ref = nf.fwd(x, g, b, **kw)
        out, call = nf.prepare_fwd(x, g, b, scales_padded=True, **kw)
        for k in ("scale_inv", "colwise_scale_inv"):
            if out[k] is not None:
                out[k].fill_(SENTINEL)
        call()
    torch.cuda.synchronize()
    return case, ref, out


@pytest.mark.parametrize("path,layout,norm,rows,hidden", [
    ("row", "rowwise", "rmsnorm", 130, 1000),
    ("row", "rowwise", "layernorm", 7, 20480),
    ("tiles", "rowwise_colwise", "rmsnorm", 300, 4104),
    ("tiles", "colwise_rowmajor", "layernorm", 200, 1000),
    ("tiles", "rowwise_colwise_rowmajor", "rmsnorm", 129, 2056),
    ("band", "rowwise_colwise", "rmsnorm", 70, 1024),
    ("general", "rowwise_colwise", "rmsnorm", 45, 1001),
    ("general", "rowwise_colwise_rowmajor", "layernorm", 33, 130),
])
def test_fwd_mxfp8_scales_padded(path, layout, norm, rows, hidden):
    case, ref, out = _padded_case(path, layout, norm, rows, hidden)
    nb_r, nb_c = (hidden + 31) // 32, (rows + 31) // 32
    rup = lambda a, m: (a + m - 1) // m * m
    checks_made = 0
    for k, logical in (("scale_inv", (rows, nb_r)),
                       ("colwise_scale_inv", (nb_c, hidden) if layout.endswith("_rowmajor") else (hidden, nb_c))):
        if ref[k] is None:
            continue
        got = out[k].cpu().numpy()
        blocks_first = k == "colwise_scale_inv" and layout.endswith("_rowmajor")
        want_shape = ((rup(logical[0], 4), rup(logical[1], 128)) if blocks_first
                      else (rup(logical[0], 128), rup(logical[1], 4)))
        assert got.shape == want_shape, (k, got.shape, want_shape)
        a, c = logical
        assert np.array_equal(got[:a, :c], ref[k].cpu().numpy()), k
        pad = np.ones(got.shape, dtype=bool)
        pad[:a, :c] = False
        assert np.all(got[pad] == SENTINEL), k
        checks_made += 1
    assert checks_made == (2 if "colwise" in layout and layout.startswith("rowwise") else 1)
    for k in ("y", "y_colwise"):
        if ref[k] is not None:
            assert torch.equal(out[k], ref[k]), k
    # and against the oracle on the logical region
    if path == "tiles" and layout == "rowwise_colwise":
        r = oracle_fwd(case, norm, "bf16", "f32", False)
        checks.check_mx_rows(bits(out["y"]), out["scale_inv"].cpu().numpy()[:rows, :nb_r], r["v"], "e4m3", "mx rowwise")
        checks.check_mx_rows(bits(out["y_colwise"]), out["colwise_scale_inv"].cpu().numpy()[:hidden, :nb_c],
                             np.ascontiguousarray(r["v"].T), "e4m3", "mx colwise")
    assert_ws_clean()


@pytest.mark.parametrize("fp8", ["e4m3", "e5m2"])
@pytest.mark.parametrize("path", ["row", "tiles", "band"])
@pytest.mark.parametrize("norm,rows,hidden", [("rmsnorm", 300, 4104), ("layernorm", 45, 1000),
                                              ("rmsnorm", 130, 12288)])
def test_fwd_mxfp8_round_up_rule(fp8, path, norm, rows, hidden):
    """The round-up exponent rule on every forward path: rowwise only (row kernel), rowwise +
    columnwise through the statistics pass + tiles, and the single-pass band kernel. No code
    may saturate, and codes and bytes match the oracle under the same rule."""
    case = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=rows + 3 * hidden)
    # spread the block maxima over many binades so that both rules' decisions vary
    case["x"] = case["x"] * torch.exp(torch.linspace(-6.0, 6.0, rows))[:, None].to(case["x"].dtype)
    ref = oracle_fwd(case, norm, "bf16", "f32", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    layout = "rowwise" if path == "row" else "rowwise_colwise"
    with env(NORMFP8_COL_KERNEL=0 if path == "band" else 1):
        out = nf.fwd(x, g, b, norm=norm, eps=EPS, scaling="mxfp8_ceil", fp8=fp8, layout=layout)
    t = ln_terms(case, ref, norm)
    checks.check_mx_rows(bits(out["y"]), bits(out["scale_inv"]), ref["v"], fp8, "mx rowwise", terms=t,
                         rule="ceil")
    if layout != "rowwise":
        checks.check_mx_rows(bits(out["y_colwise"]), bits(out["colwise_scale_inv"]),
                             np.ascontiguousarray(ref["v"].T), fp8, "mx colwise", terms=T(t), rule="ceil")
    # the rules really differ on this input
    fl = nf.fwd(x, g, b, norm=norm, eps=EPS, scaling="mxfp8", fp8=fp8, layout="rowwise")
    assert int((bits(fl["scale_inv"]) != bits(out["scale_inv"])).sum()) > 0
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                       out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    assert_ws_clean()


def test_fwd_mxfp8_zero_block():
    case = workloads.small_case("layernorm", 32, 256, "bf16", "f32", seed=4)
    case["gamma"][:32] = 0.0                          # first column block of every row is 0 * x + beta
    case["beta"][:32] = 0.0
    ref = oracle_fwd(case, "layernorm", "bf16", "f32", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    out = nf.fwd(x, g, b, norm="layernorm", scaling="mxfp8", layout="rowwise_colwise")
    sc = bits(out["scale_inv"])
    assert np.all(sc[:, 0] == 0) and np.all(bits(out["y"])[:, :32] == 0)
    checks.check_mx_rows(bits(out["y_colwise"]), bits(out["colwise_scale_inv"]),
                         np.ascontiguousarray(ref["v"].T), "e4m3", "mx colwise", terms=T(ln_terms(case, ref, "layernorm")))


# ------------------------------------------------------------------------------ columnwise tiles

# (rows, hidden): one tile, ragged rows (N % 16 != 0 and N % 128 != 0), hidden not a multiple
# of 512 or of 32, bands split over up to 40 workgroups, and sizes that enable ticket classes
COL_SHAPES = [(1, 8), (128, 512), (45, 1000), (300, 4104), (130, 8192), (2, 20480), (4096, 512),
              (4096, 2048)]


@pytest.mark.parametrize("scaling", ["delayed", "mxfp8"])
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("rows,hidden", COL_SHAPES)
def test_fwd_colwise_tiles(scaling, norm, rows, hidden):
    case = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=rows * 7 + hidden)
    ref = oracle_fwd(case, norm, "bf16", "f32", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    if scaling == "delayed":
        scale = float(np.float32(448.0) / np.float32(np.max(np.abs(ref["v"]))))
        st = torch.tensor([scale], device="cuda")
        out = nf.fwd(x, g, b, norm=norm, eps=EPS, scaling="delayed", scale=st, amax=torch.zeros(1, device="cuda"),
                     layout="rowwise_colwise")
        got = {"y": bits(out["y"]), "y_colwise": bits(out["y_colwise"]), "scale_inv": out["scale_inv"].item(),
               "colwise_scale_inv": out["colwise_scale_inv"].item(), "amax": out["amax"].item()}
        checks.check_delayed(got, ref["v"], scale, 0.0, "e4m3", rowwise=True, colwise=True,
                             terms=ln_terms(case, ref, norm))
    else:
        out = nf.fwd(x, g, b, norm=norm, eps=EPS, scaling="mxfp8", layout="rowwise_colwise")
        t = ln_terms(case, ref, norm)
        checks.check_mx_rows(bits(out["y"]), bits(out["scale_inv"]), ref["v"], "e4m3", "mx rowwise", terms=t)
        checks.check_mx_rows(bits(out["y_colwise"]), bits(out["colwise_scale_inv"]),
                             np.ascontiguousarray(ref["v"].T), "e4m3", "mx colwise", terms=T(t))
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                       out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    assert_ws_clean()


@pytest.mark.parametrize("scaling", ["delayed", "mxfp8", "mxfp8_ceil"])
@pytest.mark.parametrize("layout", ["colwise_rowmajor", "rowwise_colwise_rowmajor"])
@pytest.mark.parametrize("norm,rows,hidden", [("rmsnorm", 300, 4104), ("layernorm", 45, 1000),
                                              ("rmsnorm", 256, 8192)])
def test_fwd_colwise_rowmajor(scaling, layout, norm, rows, hidden):
    """The columnwise output in the rowwise [rows, hidden] orientation: bitwise the transpose of
    the transposed layout's output on the same inputs, and against the oracle."""
    case = workloads.small_case(norm, rows, hidden, "bf16", "f32", seed=rows + hidden + 1)
    ref = oracle_fwd(case, norm, "bf16", "f32", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    kw = dict(norm=norm, eps=EPS)
    if scaling == "delayed":
        scale = float(np.float32(448.0) / np.float32(np.max(np.abs(ref["v"]))))
        kw.update(scaling="delayed", scale=torch.tensor([scale], device="cuda"))
    else:
        kw.update(scaling=scaling)
    fresh = (lambda: dict(amax=torch.zeros(1, device="cuda"))) if scaling == "delayed" else dict
    out = nf.fwd(x, g, b, layout=layout, **kw, **fresh())
    tr = nf.fwd(x, g, b, layout=layout.replace("_rowmajor", ""), **kw, **fresh())
    assert out["y_colwise"].shape == (rows, hidden)
    assert torch.equal(out["y_colwise"], tr["y_colwise"].T)
    if layout.startswith("rowwise"):
        assert torch.equal(out["y"], tr["y"])
    t = ln_terms(case, ref, norm)
    if scaling == "delayed":
        assert torch.equal(out["colwise_scale_inv"], tr["colwise_scale_inv"])
        got = {"y": None, "y_colwise": np.ascontiguousarray(bits(out["y_colwise"]).T), "scale_inv": None,
               "colwise_scale_inv": out["colwise_scale_inv"].item(), "amax": out["amax"].item()}
        checks.check_delayed(got, ref["v"], scale, 0.0, "e4m3", rowwise=False, colwise=True, terms=t)
    else:
        assert out["colwise_scale_inv"].shape == ((rows + 31) // 32, hidden)
        assert torch.equal(out["colwise_scale_inv"], tr["colwise_scale_inv"].T)
        checks.check_mx_rows(np.ascontiguousarray(bits(out["y_colwise"]).T),
                             np.ascontiguousarray(bits(out["colwise_scale_inv"]).T),
                             np.ascontiguousarray(ref["v"].T), "e4m3", "mx colwise", terms=T(t),
                             rule="ceil" if scaling == "mxfp8_ceil" else "floor")
    assert_ws_clean()


@pytest.mark.parametrize("in_dt", ["f32", "f16"])
@pytest.mark.parametrize("layout", ["colwise", "rowwise_colwise"])
def test_fwd_colwise_other_input_dtypes(in_dt, layout):
    case = workloads.small_case("layernorm", 200, 1536, in_dt, "bf16", seed=11)
    ref = oracle_fwd(case, "layernorm", in_dt, "bf16", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    out = nf.fwd(x, g, b, norm="layernorm", eps=EPS, scaling="mxfp8", fp8="e5m2", layout=layout)
    t = ln_terms(case, ref, "layernorm", "bf16")
    if layout != "colwise":
        checks.check_mx_rows(bits(out["y"]), bits(out["scale_inv"]), ref["v"], "e5m2", "mx rowwise", terms=t)
    checks.check_mx_rows(bits(out["y_colwise"]), bits(out["colwise_scale_inv"]),
                         np.ascontiguousarray(ref["v"].T), "e5m2", "mx colwise", terms=T(t))
    checks.check_stats(out["mu"].cpu().numpy(), out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    assert_ws_clean()


@pytest.mark.parametrize("classes", [1, 8])
def test_fwd_colwise_classes_and_repeats(classes):
    """Ticket classes on and off; consecutive launches reuse the workspace (tags, tickets)."""
    case = workloads.small_case("rmsnorm", 4096, 1024, "bf16", "f32", seed=5)
    ref = oracle_fwd(case, "rmsnorm", "bf16", "f32", False)
    x, g = gpu(case, "x", "gamma")
    with env(NORMFP8_BAND_CLASSES=classes):
        for _ in range(3):
            out = nf.fwd(x, g, None, norm="rmsnorm", eps=EPS, scaling="mxfp8", layout="rowwise_colwise")
            checks.check_mx_rows(bits(out["y_colwise"]), bits(out["colwise_scale_inv"]),
                                 np.ascontiguousarray(ref["v"].T), "e4m3", "mx colwise")
    assert_ws_clean()


@pytest.mark.parametrize("scaling", ["delayed", "mxfp8"])
def test_fwd_colwise_32_row_band_kernel(scaling):
    """The 32-row band kernel's columnwise path (selected with NORMFP8_COL_KERNEL=0)."""
    case = workloads.small_case("rmsnorm", 100, 2056, "bf16", "f32", seed=3)
    ref = oracle_fwd(case, "rmsnorm", "bf16", "f32", False)
    x, g = gpu(case, "x", "gamma")
    with env(NORMFP8_COL_KERNEL=0):
        if scaling == "delayed":
            scale = float(np.float32(448.0) / np.float32(np.max(np.abs(ref["v"]))))
            out = nf.fwd(x, g, None, norm="rmsnorm", eps=EPS, scaling="delayed", layout="rowwise_colwise",
                         scale=torch.tensor([scale], device="cuda"), amax=torch.zeros(1, device="cuda"))
            got = {"y": bits(out["y"]), "y_colwise": bits(out["y_colwise"]), "scale_inv": out["scale_inv"].item(),
                   "colwise_scale_inv": out["colwise_scale_inv"].item(), "amax": out["amax"].item()}
            checks.check_delayed(got, ref["v"], scale, 0.0, "e4m3", rowwise=True, colwise=True)
        else:
            out = nf.fwd(x, g, None, norm="rmsnorm", eps=EPS, scaling="mxfp8", layout="rowwise_colwise")
            checks.check_mx_rows(bits(out["y_colwise"]), bits(out["colwise_scale_inv"]),
                                 np.ascontiguousarray(ref["v"].T), "e4m3", "mx colwise")
    assert_ws_clean()


# ------------------------------------------------------------------------------ backward

def oracle_bwd(case, norm, in_dt, w_dt, zc, ref_fwd, add=False):
    return oracle.backward_stored(host_np(case["dy"], in_dt), host_np(case["x"], in_dt),
                                  ref_fwd["mu"], ref_fwd["rsigma"], host_np(case["gamma"], w_dt),
                                  norm=norm, in_dtype=in_dt, w_dtype=w_dt, zero_centered_gamma=zc,
                                  residual_dy=host_np(case["residual_dy"], in_dt) if add else None)


BWD_SHAPES = [(1, 8), (7, 1000), (64, 1024), (300, 2048), (33, 4096), (129, 8192), (5, 16384)]


@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
@pytest.mark.parametrize("rows,hidden", BWD_SHAPES)
def test_bwd(norm, in_dt, rows, hidden):
    case = workloads.small_case(norm, rows, hidden, in_dt, "f32", seed=rows * 3 + hidden)
    ref_f = oracle_fwd(case, norm, in_dt, "f32", False)
    ref = oracle_bwd(case, norm, in_dt, "f32", False, ref_f)
    dy, x, g = gpu(case, "dy", "x", "gamma")
    mu = torch.tensor(ref_f["mu"], dtype=torch.float32, device="cuda") if norm == "layernorm" else None
    rs = torch.tensor(ref_f["rsigma"], dtype=torch.float32, device="cuda")
    out = nf.bwd(dy, x, mu, rs, g, norm=norm)
    checks.check_dx(bits(out["dx"]), ref["dx"], in_dt)
    checks.check_wgrad(out["dgamma"].cpu().numpy(), ref["dgamma"])
    if norm == "layernorm":
        checks.check_wgrad(out["dbeta"].cpu().numpy(), ref["dbeta"], what="dbeta")


@pytest.mark.parametrize("cfg", range(len(BWD_COVER)))
def test_bwd_every_layout(cfg):
    hidden = BWD_COVER[cfg] - 8
    case = workloads.small_case("layernorm", 21, hidden, "bf16", "f32", seed=cfg + 5)
    ref_f = oracle_fwd(case, "layernorm", "bf16", "f32", False)
    ref = oracle_bwd(case, "layernorm", "bf16", "f32", False, ref_f)
    dy, x, g = gpu(case, "dy", "x", "gamma")
    mu = torch.tensor(ref_f["mu"], dtype=torch.float32, device="cuda")
    rs = torch.tensor(ref_f["rsigma"], dtype=torch.float32, device="cuda")
    with env(NORMFP8_BWD_CFG=cfg):
        out = nf.bwd(dy, x, mu, rs, g, norm="layernorm")
    checks.check_dx(bits(out["dx"]), ref["dx"], "bf16")
    checks.check_wgrad(out["dgamma"].cpu().numpy(), ref["dgamma"])
    checks.check_wgrad(out["dbeta"].cpu().numpy(), ref["dbeta"], what="dbeta")


@pytest.mark.parametrize("rows,hidden,zc", [(1, 8, False), (77, 2048, True), (256, 8192, False)])
def test_bwd_add(rows, hidden, zc):
    case = workloads.small_case("rmsnorm", rows, hidden, "bf16", "f32", seed=hidden + 1, zero_centered_gamma=zc)
    ref_f = oracle_fwd(case, "rmsnorm", "bf16", "f32", zc)
    ref = oracle_bwd(case, "rmsnorm", "bf16", "f32", zc, ref_f, add=True)
    dy, x, r, g = gpu(case, "dy", "x", "residual_dy", "gamma")
    rs = torch.tensor(ref_f["rsigma"], dtype=torch.float32, device="cuda")
    out = nf.bwd_add(dy, x, r, rs, g, zero_centered_gamma=zc)
    checks.check_dx(bits(out["dx"]), ref["dx"], "bf16")
    checks.check_wgrad(out["dgamma"].cpu().numpy(), ref["dgamma"])


def test_bwd_zero_rows_gives_zero_gradients():
    case = workloads.small_case("layernorm", 4, 256, "bf16", "f32", seed=1)
    dy, x, g = gpu(case, "dy", "x", "gamma")
    mu = torch.zeros(0, device="cuda")
    rs = torch.zeros(0, device="cuda")
    out = nf.bwd(dy[:0], x[:0], mu, rs, g, norm="layernorm")
    assert torch.all(out["dgamma"] == 0) and torch.all(out["dbeta"] == 0)


@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm", "rmsnorm_add"])
def test_bwd_zero_rows_with_null_row_pointers(kind):
    """rows == 0 with every row-indexed pointer NULL (allowed by the boundary): zero gradients,
    nothing read."""
    import ctypes
    from rmsnorm_fp8_quantization_amd import _lib as L, ops
    norm = "rmsnorm" if kind.startswith("rms") else "layernorm"
    add = kind == "rmsnorm_add"
    hidden = 4096
    dev = torch.device("cuda")
    g = torch.randn(hidden, device=dev)
    dg = torch.full((hidden,), 7.0, device=dev)
    db = torch.full((hidden,), 7.0, device=dev) if norm == "layernorm" else None
    ws = ops.workspace(ops.bwd_workspace_size(0, hidden, torch.bfloat16, torch.float32, norm, add), dev)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if add:
        L.call("norm_bwd_add", stream, None, None, None, None, p(g), None, p(dg), p(ws), ws.numel(), 0, hidden,
               L.NORM_BF16, L.NORM_F32, 0, 0)
    else:
        L.call("norm_bwd", stream, None, None, None, None, p(g), None, p(dg), p(db), p(ws), ws.numel(), 0, hidden,
               L.NORM_BF16, L.NORM_F32, L.NORM_LAYERNORM if norm == "layernorm" else L.NORM_RMSNORM, 0, 0)
    torch.cuda.synchronize()
    assert torch.all(dg == 0)
    if db is not None:
        assert torch.all(db == 0)


def test_fwd_then_bwd_end_to_end():
    """GPU statistics feeding the GPU backward, against the oracle with its own statistics."""
    case = workloads.small_case("layernorm", 128, 4096, "bf16", "f32", seed=77)
    ref_f = oracle_fwd(case, "layernorm", "bf16", "f32", False)
    ref = oracle_bwd(case, "layernorm", "bf16", "f32", False, ref_f)
    dy, x, g, b = gpu(case, "dy", "x", "gamma", "beta")
    f = nf.fwd(x, g, b, norm="layernorm")
    out = nf.bwd(dy, x, f["mu"], f["rsigma"], g, norm="layernorm")
    checks.check_dx(bits(out["dx"]), ref["dx"], "bf16")
    checks.check_wgrad(out["dgamma"].cpu().numpy(), ref["dgamma"])


# ------------------------------------------------------------------------------ split rows

SPLIT_SHAPES = [(3, 8), (5, 4096), (37, 16384), (9, 16392), (300, 40000), (2, 65536), (70, 65536),
                (4, 131072), (1, 98304), (520, 65536), (3, 196608), (2, 262144)]


@pytest.mark.parametrize("shape", [0, 1, 2])
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("in_dt", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("rows,hidden", SPLIT_SHAPES)
def test_fwd_split_rows(norm, in_dt, rows, hidden, shape):
    """The split kernel (S = ceil(hidden / W) workgroups per row, tagged partial exchange),
    forced on every shape: one to eight slices, ragged last slices, fewer rows than row groups
    and several rows per group (rows needing more than eight slices of the forced shape go to
    the band or general kernels). Shape 0: 16384-column slices with the weights in LDS, four rows
    in flight; shapes 1 and 2 (16-bit input; float32 input stays on shape 0): 32768- or
    16384-column slices with gamma in registers and beta in LDS, three or four rows in flight."""
    case = workloads.small_case(norm, rows, hidden, in_dt, "f32", seed=rows + hidden + 11)
    ref = oracle_fwd(case, norm, in_dt, "f32", False)
    x, g, b = gpu(case, "x", "gamma", "beta")
    print(f"split: shape {shape} {norm} {in_dt} {rows}x{hidden}", flush=True)
    with env(NORMFP8_SPLIT=1, NORMFP8_SPLIT_SHAPE=shape):
        out = nf.fwd(x, g, b, norm=norm, eps=EPS)
    checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                       out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
    checks.check_hp(bits(out["y"]), ref["v"], in_dt, terms=ln_terms(case, ref, norm))
    assert_ws_clean()


@pytest.mark.parametrize("shape", [0, 1, 2])
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_fwd_split_zero_centered_bf16_weights_and_margin(norm, shape):
    rows, hidden = 33, 49152
    case = workloads.small_case(norm, rows, hidden, "bf16", "bf16", seed=5, zero_centered_gamma=True)
    ref = oracle_fwd(case, norm, "bf16", "bf16", True)
    x, g, b = gpu(case, "x", "gamma", "beta")
    for margin in (0, 200, 250):
        with env(NORMFP8_SPLIT=1, NORMFP8_SPLIT_SHAPE=shape):
            out = nf.fwd(x, g, b, norm=norm, eps=EPS, zero_centered_gamma=True, cu_margin=margin)
        checks.check_stats(out["mu"].cpu().numpy() if out["mu"] is not None else None,
                           out["rsigma"].cpu().numpy(), ref["mu"], ref["rsigma"])
        checks.check_hp(bits(out["y"]), ref["v"], "bf16", terms=ln_terms(case, ref, norm, "bf16", zc=True))
    assert_ws_clean()


# ------------------------------------------------------------------------------ single-pass columnwise

# (rows, hidden, cu_margin): 1 to 24 slices of 512 columns; margins that leave one or two groups
# of slices walking many 128-row super-bands (2 to 18 pipeline steps; step counts of 4k and 4k + 2
# end the four-band rotation at either of its two exits)
COLX_SHAPES = [(128, 512, 0), (256, 1536, 0), (384, 4096, 0), (128, 12288, 0), (1024, 2048, 250),
               (640, 8192, 240), (768, 4096, 0), (1152, 1024, 254), (1920, 1024, 252)]


def _colx_planned(rows, hidden, in_dt, scaling, layout, margin):
    """The single-pass kernel's row partials (rows x slices tagged words) are in the workspace
    plan when it is chosen."""
    kw = dict(rows=rows, hidden=hidden, in_dtype=TDT[in_dt], w_dtype=torch.float32, out_code=nf._lib.NORM_FP8_E4M3,
              norm="rmsnorm", scaling=scaling, layout=layout, cu_margin=margin)
    with env(NORMFP8_COLX=1):
        on = nf.fwd_workspace_size(**kw)
    with env(NORMFP8_COLX=0):
        off = nf.fwd_workspace_size(**kw)
    return on >= off + rows * (hidden // 512) * 8


def _colx_check(case, out, scaling, fp8, layout, in_dt="bf16", w_dt="f32", zc=False, scale=None):
    ref = oracle_fwd(case, "rmsnorm", in_dt, w_dt, zc)
    if scaling == "delayed":
        got = {"y": bits(out["y"]) if out["y"] is not None else None, "y_colwise": bits(out["y_colwise"]),
               "scale_inv": out["scale_inv"].item() if out["scale_inv"] is not None else None,
               "colwise_scale_inv": out["colwise_scale_inv"].item(), "amax": out["amax"].item()}
        checks.check_delayed(got, ref["v"], scale, 0.25, fp8, rowwise=layout != "colwise", colwise=True)
    else:
        rule = "ceil" if scaling == "mxfp8_ceil" else "floor"
        if layout != "colwise":
            checks.check_mx_rows(bits(out["y"]), bits(out["scale_inv"]), ref["v"], fp8, "mx rowwise", rule=rule)
        checks.check_mx_rows(bits(out["y_colwise"]), bits(out["colwise_scale_inv"]),
                             np.ascontiguousarray(ref["v"].T), fp8, "mx colwise", rule=rule)
    checks.check_stats(None, out["rsigma"].cpu().numpy(), None, ref["rsigma"])


def _colx_kw(case, scaling, fp8, ref_max):
    if scaling != "delayed":
        return {"scaling": scaling, "fp8": fp8}, None
    top = F.E4M3.max_finite if fp8 == "e4m3" else F.E5M2.max_finite
    scale = float(np.float32(top) / np.float32(ref_max / 4))    # a quarter of the range saturates
    return {"scaling": "delayed", "fp8": fp8, "scale": torch.tensor([scale], device="cuda"),
            "amax": torch.tensor([0.25], device="cuda")}, scale


@pytest.mark.parametrize("scaling", ["delayed", "mxfp8", "mxfp8_ceil"])
@pytest.mark.parametrize("layout", ["rowwise_colwise", "colwise"])
@pytest.mark.parametrize("rows,hidden,margin", COLX_SHAPES)
def test_fwd_colx(scaling, layout, rows, hidden, margin):
    """RMSNorm with a columnwise FP8 output in one pass over x (bands of 128 rows, slices of 512
    columns exchanging row sums of squares), forced, against the oracle."""
    case = workloads.small_case("rmsnorm", rows, hidden, "bf16", "f32", seed=rows * 7 + hidden + margin)
    xh = case["x"].float()
    xh[::5, ::11] *= 16.0                        # outliers: saturated codes, spread block scales
    case["x"] = xh.to(torch.bfloat16)
    assert _colx_planned(rows, hidden, "bf16", scaling, layout, margin)
    ref_max = float(np.max(np.abs(oracle_fwd(case, "rmsnorm", "bf16", "f32", False)["v"])))
    kw, scale = _colx_kw(case, scaling, "e4m3", ref_max)
    x, g = gpu(case, "x", "gamma")
    with env(NORMFP8_COLX=1):
        out = nf.fwd(x, g, None, norm="rmsnorm", eps=EPS, layout=layout, cu_margin=margin, **kw)
    _colx_check(case, out, scaling, "e4m3", layout, scale=scale)
    assert_ws_clean()


@pytest.mark.parametrize("scaling", ["delayed", "mxfp8"])
@pytest.mark.parametrize("variant", ["e5m2", "f16", "bf16_weights_zc", "padded"])
def test_fwd_colx_variants(scaling, variant):
    """The single-pass kernel with E5M2 codes, float16 input, bfloat16 zero-centred weights, and
    (MXFP8) padded scale grids whose padding stays as the caller filled it."""
    rows, hidden = 512, 3072
    in_dt = "f16" if variant == "f16" else "bf16"
    w_dt = "bf16" if variant == "bf16_weights_zc" else "f32"
    zc = variant == "bf16_weights_zc"
    fp8 = "e5m2" if variant == "e5m2" else "e4m3"
    if variant == "padded" and scaling == "delayed":
        pytest.skip("padded grids are MXFP8's")
    case = workloads.small_case("rmsnorm", rows, hidden, in_dt, w_dt, seed=31, zero_centered_gamma=zc)
    assert _colx_planned(rows, hidden, in_dt, scaling, "rowwise_colwise", 0)
    ref_max = float(np.max(np.abs(oracle_fwd(case, "rmsnorm", in_dt, w_dt, zc)["v"])))
    kw, scale = _colx_kw(case, scaling, fp8, ref_max)
    x, g = gpu(case, "x", "gamma")
    with env(NORMFP8_COLX=1):
        if variant == "padded":
            out, call = nf.prepare_fwd(x, g, None, norm="rmsnorm", eps=EPS, layout="rowwise_colwise",
                                       scales_padded=True, **kw)
            for k in ("scale_inv", "colwise_scale_inv"):
                out[k].fill_(SENTINEL)
            call()
            torch.cuda.synchronize()
            for k, (a, c) in (("scale_inv", (rows, hidden // 32)), ("colwise_scale_inv", (hidden, rows // 32))):
                pad = out[k].clone()
                pad[:a, :c] = SENTINEL
                assert bool((pad == SENTINEL).all()), f"{k}: padding written"
                out[k] = out[k][:a, :c].contiguous()
        else:
            out = nf.fwd(x, g, None, norm="rmsnorm", eps=EPS, zero_centered_gamma=zc, layout="rowwise_colwise", **kw)
    _colx_check(case, out, scaling, fp8, "rowwise_colwise", in_dt, w_dt, zc, scale)
    assert_ws_clean()


def test_fwd_colx_matches_two_pass_statistics():
    """The single-pass kernel's rsigma (slice partials summed in one fixed order) agrees with the
    two-pass route's to a few ulps, and both kernels' codes differ only where the oracle allows."""
    rows, hidden = 1024, 6144
    case = workloads.small_case("rmsnorm", rows, hidden, "bf16", "f32", seed=77)
    x, g = gpu(case, "x", "gamma")
    outs = {}
    for k in (0, 1):
        with env(NORMFP8_COLX=k):
            outs[k] = nf.fwd(x, g, None, norm="rmsnorm", eps=EPS, scaling="mxfp8", layout="rowwise_colwise")
    a, b = outs[0]["rsigma"].cpu().numpy(), outs[1]["rsigma"].cpu().numpy()
    assert np.max(np.abs(a - b) / np.abs(a)) < 4 * 2.0 ** -23
    for k in (0, 1):
        _colx_check(case, outs[k], "mxfp8", "e4m3", "rowwise_colwise")


# ------------------------------------------------------------------------------ determinism

def test_repeat_runs_are_bitwise_identical():
    """Repeated calls give the same bytes: the band split (forced: its cross-workgroup exchange
    of row partials through tagged words and tickets), both split kernel shapes, the columnwise tile path,
    the single-pass columnwise band kernel, the single-pass RMSNorm columnwise kernel (row sums
    exchanged between 512-column slices; MXFP8 and delayed) and the backward's fixed-order partial
    reduction."""
    case = workloads.small_case("layernorm", 500, 20480, "bf16", "f32", seed=8)
    dy, x, g, b = gpu(case, "dy", "x", "gamma", "beta")
    xs, dys, gs = x[:, :16384].contiguous(), dy[:, :16384].contiguous(), g[:16384].contiguous()
    xr, gr = x[:384, :6144].contiguous(), g[:6144].contiguous()   # 3 super-bands x 12 slices
    wide = workloads.small_case("layernorm", 300, 40000, "bf16", "f32", seed=9)
    xw, gw, bw = gpu(wide, "x", "gamma", "beta")
    st = torch.tensor([16.0], device="cuda")
    outs = []
    for _ in range(3):
        with env(NORMFP8_COLX=1):
            fm = nf.fwd(xr, gr, None, norm="rmsnorm", scaling="mxfp8", layout="rowwise_colwise")
            fd = nf.fwd(xr, gr, None, norm="rmsnorm", scaling="delayed", scale=st,
                        amax=torch.zeros(1, device="cuda"), layout="rowwise_colwise")
        outs_x = [fm["y"], fm["y_colwise"], fm["scale_inv"], fm["colwise_scale_inv"], fm["rsigma"],
                  fd["y"], fd["y_colwise"], fd["amax"], fd["rsigma"]]
        with env(NORMFP8_FORCE_BAND=1, NORMFP8_SPLIT=0):
            f = nf.fwd(x, g, b, norm="layernorm")                  # band split (20480 columns)
        with env(NORMFP8_SPLIT=1, NORMFP8_SPLIT_SHAPE=0):
            fs = nf.fwd(x, g, b, norm="layernorm")                 # split kernel (two slices)
        with env(NORMFP8_SPLIT=1, NORMFP8_SPLIT_SHAPE=1):
            fs1 = nf.fwd(xw, gw, bw, norm="layernorm")             # 8-wave split shape (two slices)
        with env(NORMFP8_SPLIT=1, NORMFP8_SPLIT_SHAPE=2):
            fs2 = nf.fwd(xw, gw, bw, norm="layernorm")             # 16384-column 8-wave shape (three slices)
        with env(NORMFP8_COL_KERNEL=0):
            fb = nf.fwd(x, g, b, norm="layernorm", scaling="mxfp8", layout="rowwise_colwise")
        fc = nf.fwd(x, g, b, norm="layernorm", scaling="mxfp8", layout="rowwise_colwise")
        d = nf.bwd(dys, xs, f["mu"], f["rsigma"], gs, norm="layernorm")
        outs.append([t.clone() for t in (f["y"], f["mu"], f["rsigma"], fs["y"], fs["mu"], fs["rsigma"],
                                          fs1["y"], fs1["mu"], fs1["rsigma"], fs2["y"], fs2["mu"], fs2["rsigma"],
                                          fb["y"], fb["y_colwise"], fb["rsigma"],
                                          fc["y"], fc["y_colwise"], fc["colwise_scale_inv"],
                                          d["dx"], d["dgamma"], d["dbeta"], *outs_x)])
    for o in outs[1:]:
        for a, b_ in zip(outs[0], o):
            assert torch.equal(a.view(torch.uint8), b_.view(torch.uint8))
    assert_ws_clean()
