"""The forward planner's choice of kernels and launch layout, queried on the host (no GPU).

``norm_fwd_launch_shape`` returns what ``norm_fwd`` would launch for a request: the route (row
kernel, row kernel + byte transpose, statistics pass + tiles, band, split, single-pass columnwise,
general), the layout and, for a row layout, its waves per row (P), 16-byte strips per lane (KC)
and rows per workgroup (T). These tests pin the measured choices the planner documents for each
row length, norm, input dtype and epilogue, so a change to the preference lists or their
exceptions shows up here before a GPU run. The parity of every layout is covered by the GPU tests;
this file checks only which layout a request gets.

[NVRTC-PR] "Migrate norms and softmax kernels to NVRTC", Description and Flowchart: tuned
kernels chosen per row length, a general kernel for every other size.
"""
import ctypes
import os

import pytest

L = pytest.importorskip("rmsnorm_fp8_quantization_amd._lib")

LN, RMS = L.NORM_LAYERNORM, L.NORM_RMSNORM
BF16, F16, F32, E4M3 = L.NORM_BF16, L.NORM_F16, L.NORM_F32, L.NORM_FP8_E4M3
PLAIN, DELAYED, MX = L.NORM_SCALING_NONE, L.NORM_SCALING_DELAYED_TENSOR, L.NORM_SCALING_MXFP8_1D32
ROW, BOTH, COL = L.NORM_Q_ROWWISE, L.NORM_Q_ROWWISE_COLWISE, L.NORM_Q_COLWISE

# row layouts by (waves per row P, strips per lane KC, rows per workgroup T)
W1_K1, W1_K2, W1_K4 = (1, 1, 4), (1, 2, 4), (1, 4, 4)
W2T2_K4, W4_K4, W8_K4 = (2, 4, 2), (4, 4, 1), (8, 4, 1)
W4T2_K2, W4T4_K4, W8T2_K4 = (4, 2, 2), (4, 4, 4), (8, 4, 2)
W16_K2, W16_K4, W16_K8 = (16, 2, 1), (16, 4, 1), (16, 8, 1)
W8_K8, W4_K8 = (8, 8, 1), (4, 8, 1)


def _lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libnormfp8.so not built (run __graft_entry__.build())")
    return L.load()


def plan(rows, hidden, norm, in_dt=BF16, out_dt=None, scaling=PLAIN, qlayout=ROW, w_dt=F32, margin=0):
    _lib()
    if out_dt is None:
        out_dt = E4M3 if scaling != PLAIN else in_dt
    shape = (ctypes.c_int64 * 6)()
    L.call("norm_fwd_launch_shape", rows, hidden, in_dt, w_dt, out_dt, norm, scaling, qlayout, margin, shape)
    return tuple(int(v) for v in shape)


def row_layout(shape):
    assert shape[0] in (L.NORM_ROUTE_ROW, L.NORM_ROUTE_ROW_TRANSPOSE, L.NORM_ROUTE_STATS_TILES), shape
    return shape[2:5]


# (norm, input dtype, hidden) -> the row layout of a plain (no FP8) forward
PLAIN_CASES = [
    (LN, BF16, 256, W1_K1), (LN, BF16, 512, W1_K1), (LN, BF16, 1024, W1_K2), (LN, BF16, 2048, W1_K4),
    (LN, BF16, 4096, W2T2_K4), (LN, BF16, 8192, W4T4_K4),
    # LayerNorm 8193..16384, 16-bit input: gamma and beta in registers on 4 waves
    (LN, BF16, 8200, W4_K8), (LN, BF16, 12288, W4_K8), (LN, F16, 16384, W4_K8),
    # ... float32 input keeps two rows of 8 waves sharing the LDS weights
    (LN, F32, 12288, W8T2_K4), (LN, F32, 16384, W8T2_K4),
    # LayerNorm 16385..32768, 16-bit input: 8 waves with the weights in registers
    (LN, BF16, 16392, W8_K8), (LN, BF16, 20480, W8_K8), (LN, F16, 32768, W8_K8),
    (LN, F32, 20480, W16_K4),
    (LN, F32, 32776, W16_K8), (LN, F32, 40960, W16_K8),
    (RMS, BF16, 256, W1_K1), (RMS, BF16, 4096, W2T2_K4), (RMS, BF16, 8192, W4_K4),
    (RMS, BF16, 12288, W16_K2), (RMS, BF16, 16384, W16_K2),
    (RMS, BF16, 20480, W16_K4), (RMS, F32, 32768, W16_K4), (RMS, BF16, 40960, W16_K8),
    (RMS, BF16, 65536, W16_K8), (LN, F32, 65536, W16_K8),
]


@pytest.mark.parametrize("norm,in_dt,hidden,layout", PLAIN_CASES)
def test_plain_forward_row_layout_per_width(norm, in_dt, hidden, layout):
    s = plan(1000, hidden, norm, in_dt)
    assert s[0] == L.NORM_ROUTE_ROW, s
    assert row_layout(s) == layout
    assert s[5] == 1
    # a row layout covers the row with its waves x strips x 512 elements
    assert 512 * layout[0] * layout[1] >= hidden


@pytest.mark.parametrize("scaling", [DELAYED, MX])
def test_fp8_rowwise_row_layouts(scaling):
    # RMSNorm with 1-byte codes: four rows per workgroup at 4097..8192, 8 waves x 4 strips at
    # 8193..16384, 4 waves x 2 rows x 2 strips at 2049..4096
    assert row_layout(plan(1000, 8192, RMS, scaling=scaling)) == W4T4_K4
    assert row_layout(plan(1000, 12288, RMS, scaling=scaling)) == W8_K4
    assert row_layout(plan(1000, 10240, RMS, scaling=scaling)) == W8_K4
    assert row_layout(plan(1000, 4096, RMS, scaling=scaling)) == W4T2_K2
    # ... while a 2-byte plain output keeps one row per workgroup at 8192
    assert row_layout(plan(1000, 8192, RMS)) == W4_K4
    # LayerNorm FP8 epilogues keep the LDS-weight layouts (no register-weight instances for them)
    assert row_layout(plan(1000, 12288, LN, scaling=scaling)) == W8T2_K4
    assert row_layout(plan(1000, 20480, LN, scaling=scaling)) == W16_K4


def test_delayed_both_outputs_take_the_transpose_route():
    for norm in (LN, RMS):
        s = plan(1000, 8192, norm, scaling=DELAYED, qlayout=BOTH)
        assert s[0] == L.NORM_ROUTE_ROW_TRANSPOSE, s
        # the columnwise request keeps the default layout, so both routes reduce each row alike
        assert row_layout(s) == W4T4_K4
    # a width that is not a multiple of 16 has no byte transpose: statistics + tiles
    s = plan(1000, 8200, LN, scaling=DELAYED, qlayout=BOTH)
    assert s[0] == L.NORM_ROUTE_STATS_TILES, s


def test_mxfp8_columnwise_takes_statistics_and_tiles_for_layernorm():
    s = plan(1000, 8192, LN, scaling=MX, qlayout=BOTH)
    assert s[0] == L.NORM_ROUTE_STATS_TILES and row_layout(s) == W4T4_K4
    s = plan(1000, 1024, LN, scaling=MX, qlayout=COL)
    assert s[0] == L.NORM_ROUTE_STATS_TILES and row_layout(s) == W1_K2


@pytest.mark.parametrize("rows,hidden,scaling,qlayout,S", [
    (16384, 12288, MX, BOTH, 24), (32768, 8192, DELAYED, BOTH, 16), (128, 512, MX, COL, 1),
    (256, 4096, MX, COL, 8),
])
def test_rmsnorm_fp8_columnwise_single_pass(rows, hidden, scaling, qlayout, S):
    s = plan(rows, hidden, RMS, scaling=scaling, qlayout=qlayout)
    assert s == (L.NORM_ROUTE_SINGLE_PASS_COLWISE, 0, 0, 0, 0, S)
    assert S == hidden // 512


def test_single_pass_columnwise_conditions():
    # rows not a multiple of 128, float32 input, LayerNorm or the row-major columnwise layout
    # keep the two-pass routes
    assert plan(1000, 8192, RMS, scaling=MX, qlayout=BOTH)[0] == L.NORM_ROUTE_STATS_TILES
    assert plan(1024, 8192, RMS, F32, scaling=MX, qlayout=BOTH)[0] == L.NORM_ROUTE_STATS_TILES
    assert plan(1024, 8192, LN, scaling=MX, qlayout=BOTH)[0] == L.NORM_ROUTE_STATS_TILES
    assert plan(1024, 8192, RMS, scaling=MX, qlayout=BOTH | L.NORM_Q_COLWISE_ROWMAJOR)[0] == L.NORM_ROUTE_STATS_TILES
    # nor does a width that is not a multiple of 512
    assert plan(1024, 8200, RMS, scaling=MX, qlayout=BOTH)[0] == L.NORM_ROUTE_STATS_TILES


@pytest.mark.parametrize("norm,in_dt,hidden,shape,S", [
    # LayerNorm, 16-bit input: 8 waves with gamma in registers, 16384-column slices from 32769 to
    # 49152 elements, 32768-column slices beyond
    (LN, BF16, 32776, 2, 3), (LN, BF16, 40960, 2, 3), (LN, F16, 49152, 2, 3),
    (LN, BF16, 49160, 1, 2), (LN, BF16, 65536, 1, 2), (LN, F16, 65544, 1, 3), (LN, BF16, 262144, 1, 8),
    # RMSNorm, 16-bit input: the same shapes from 65537, 16384-column slices up to 131072
    (RMS, BF16, 65544, 2, 5), (RMS, F16, 131072, 2, 8), (RMS, BF16, 131080, 1, 5), (RMS, BF16, 262144, 1, 8),
    # float32 input: 16 waves x 2 strips with the weights in LDS, beyond 65536
    (LN, F32, 65544, 0, 5), (LN, F32, 98304, 0, 6), (RMS, F32, 131072, 0, 8),
])
def test_long_rows_take_the_split_kernel(norm, in_dt, hidden, shape, S):
    s = plan(1000, hidden, norm, in_dt)
    assert s == (L.NORM_ROUTE_SPLIT, shape, 0, 0, 0, S)
    cols = 32768 if shape == 1 else 16384  # columns one workgroup's slice holds
    assert (S - 1) * cols < hidden <= S * cols


def test_split_threshold_edges():
    assert plan(1000, 32768, LN)[0] == L.NORM_ROUTE_ROW
    assert plan(1000, 32776, LN)[0] == L.NORM_ROUTE_SPLIT
    assert plan(1000, 65536, LN, F32)[0] == L.NORM_ROUTE_ROW
    assert plan(1000, 65536, RMS)[0] == L.NORM_ROUTE_ROW
    assert plan(1000, 65544, RMS)[0] == L.NORM_ROUTE_SPLIT
    # an FP8 epilogue never takes the split kernel
    assert plan(1000, 49152, LN, scaling=DELAYED)[0] == L.NORM_ROUTE_ROW


def test_band_kernel_beyond_the_row_and_split_layouts():
    # plain rows beyond what 8 split slices hold: band tiles of 8 rows x 4096 columns
    s = plan(200, 200000, LN, F32)
    assert s == (L.NORM_ROUTE_BAND, 4, 0, 0, 0, 49)
    # beyond eight 32768-column slices and 64 band slices of 4096 columns: the general kernels
    assert plan(200, 262152, RMS) == (L.NORM_ROUTE_GENERAL, 0, 0, 0, 0, 1)
    # an FP8 rowwise epilogue beyond 65536 (no row layout covers it, no split for FP8)
    s = plan(200, 100000, RMS, scaling=DELAYED)
    assert s == (L.NORM_ROUTE_BAND, 4, 0, 0, 0, 25)


@pytest.mark.parametrize("rows,hidden,kw", [
    (1000, 4097, {}), (1000, 4100, {}), (1000, 300000, {"in_dt": F32}), (1000, 1000000, {}),
    # a columnwise output of rows longer than a band merges (64 slices of 1024 columns)
    (1000, 70000, {"scaling": MX, "qlayout": BOTH}),
])
def test_general_kernels_for_every_other_size(rows, hidden, kw):
    s = plan(rows, hidden, RMS, **kw)
    assert s == (L.NORM_ROUTE_GENERAL, 0, 0, 0, 0, 1)


def test_zero_rows_plan_like_any_other_count():
    assert plan(0, 4096, LN) == plan(1000, 4096, LN)


def test_invalid_arguments_are_rejected():
    _lib()
    shape = (ctypes.c_int64 * 6)()
    with pytest.raises(L.NormError):
        L.call("norm_fwd_launch_shape", 16, 0, BF16, F32, BF16, LN, PLAIN, ROW, 0, shape)
    with pytest.raises(L.NormError):
        L.call("norm_fwd_launch_shape", 16, 4096, BF16, F32, BF16, LN, PLAIN, ROW, 0, None)
