// api.cpp -- the C ABI declared in include/normfp8.h: argument validation, the launch planner
// and the kernel launches.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization";
// [NVRTC-PR] = "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request).
// [XLA-Norm] Description: workspace-size queries for forward and backward, a forward entry that
// takes the input / weight / scaling buffers and writes the outputs, and an SM margin removed
// from the device's multiprocessor count when sizing the launch. [NVRTC-PR] Flowchart: grid
// sizes come from occupancy, multi-CTA rows use a workspace and barrier, and the backward
// launches a finalize kernel after the partial weight-gradient kernel.
//
// MI355X design: every kernel is compiled ahead of time for gfx950 (no runtime compilation);
// the planner picks one of three forward layouts (wave / workgroup team per row, or band tiles
// with a cross-workgroup statistics exchange) from the row length and the requested outputs,
// and the backward's persistent grid from the CU count less the margin. The planner never
// reads device memory and never allocates.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

#include "../../include/normfp8.h"
#include "kernels.hpp"
#include "plan.hpp"

static_assert(NORM_WS_HEADER_BYTES == nf8::kWsHeaderBytes, "workspace header size mismatch");

namespace {

using namespace nf8;

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
int ok() {
  g_err.clear();
  return NORM_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is_hp(int dt) { return dt == DT_F32 || dt == DT_F16 || dt == DT_BF16; }
bool is_fp8(int dt) { return dt == DT_E4M3 || dt == DT_E5M2; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// ---------------------------------------------------------------- tuning knobs
// Planner overrides for testing and tuning. Each starts from the process environment, read once
// (on the library's first use); afterwards only norm_tuning_set changes them. A launch reads
// them with one relaxed atomic load each.
constexpr int kKnobUnset = INT_MIN;
const char *const kKnobNames[] = {"NORMFP8_FORCE_BAND",       "NORMFP8_ROW_CFG",      "NORMFP8_COL_KERNEL",
                                  "NORMFP8_DELAYED_TRANSPOSE", "NORMFP8_BAND_CFG",     "NORMFP8_BWD_CFG",
                                  "NORMFP8_ROW_OCC",           "NORMFP8_ROW_BALANCE",  "NORMFP8_TRANSPOSE_TC",
                                  "NORMFP8_TRANSPOSE_RL",      "NORMFP8_BAND_CLASSES", "NORMFP8_SPLIT", "NORMFP8_COLX",
                                  "NORMFP8_SPLIT_SHAPE"};
enum Knob : int {
  K_FORCE_BAND = 0,
  K_ROW_CFG,
  K_COL_KERNEL,
  K_DELAYED_TRANSPOSE,
  K_BAND_CFG,
  K_BWD_CFG,
  K_ROW_OCC,
  K_ROW_BALANCE,
  K_TRANSPOSE_TC,
  K_TRANSPOSE_RL,
  K_BAND_CLASSES,
  K_SPLIT,
  K_COLX,
  K_SPLIT_SHAPE,
  K_NKNOBS
};
static_assert(sizeof(kKnobNames) / sizeof(kKnobNames[0]) == K_NKNOBS, "knob table");
std::atomic<int> g_knobs[K_NKNOBS];
std::once_flag g_knobs_once;

void knobs_init() {
  std::call_once(g_knobs_once, [] {
    for (int i = 0; i < K_NKNOBS; ++i) {
      const char *v = getenv(kKnobNames[i]);
      g_knobs[i].store(v && *v ? atoi(v) : kKnobUnset, std::memory_order_relaxed);
    }
  });
}
int knob(Knob k, int dflt) {
  knobs_init();
  const int v = g_knobs[k].load(std::memory_order_relaxed);
  return v == kKnobUnset ? dflt : v;
}

// ---------------------------------------------------------------- device facts (cached)
struct DeviceInfo {
  int cus = 0;
};
std::mutex g_mu;
std::unordered_map<int, DeviceInfo> g_dev;
std::unordered_map<const void *, int> g_occ;  // kernel -> max resident workgroups per CU

int device_info(DeviceInfo *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NORM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_dev.find(dev);
  if (it == g_dev.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(NORM_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    DeviceInfo d;
    d.cus = prop.multiProcessorCount;
    it = g_dev.emplace(dev, d).first;
  }
  *out = it->second;
  return NORM_OK;
}

int occupancy(const void *fn, int threads, int *out) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_occ.find(fn);
    if (it != g_occ.end()) {
      *out = it->second;
      return NORM_OK;
    }
  }
  int n = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, 0);
  if (e != hipSuccess) return fail(NORM_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
  if (n < 1) n = 1;
  std::lock_guard<std::mutex> lk(g_mu);
  g_occ[fn] = n;
  *out = n;
  return NORM_OK;
}

int launch(const void *fn, dim3 grid, dim3 block, void *param, hipStream_t stream) {
  void *args[] = {param};
  hipError_t e = hipLaunchKernel(fn, grid, block, args, 0, stream);
  if (e != hipSuccess) return fail(NORM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return NORM_OK;
}

// ---------------------------------------------------------------- forward plan
struct FwdPlan {
  int mode = MODE_PLAIN;
  bool rowwise = true, colwise = false;
  bool band = false;
  bool col = false;   // columnwise output in two passes: statistics (row kernel), then tiles
  int cfg = 0;        // row layout (row path and the statistics pass) or band layout
  int tile_rows = 0;  // rows per band
  int S = 1;
  int64_t bands = 0;
  size_t ws_bytes = 0;
  size_t partial_off = 0;
  size_t colx_off = 0;   // single-pass columnwise partials
  size_t stats_off = 0;  // two-pass path: mu / rsigma when the caller passes none
  bool col_rowmajor = false;
  bool scales_padded = false;  // MXFP8 E8M0 grids padded (block dimension to 4, the other to 128)
  bool tr = false;    // delayed scaling, rowwise + columnwise: row kernel, then a byte transpose
  bool gen = false;   // general kernels: hidden not a multiple of 8 (or, at launch, unaligned tensors)
  bool split = false; // long rows, no FP8 epilogue: the split kernel (S slices per row)
  int split_shape = 0; // the split kernel's shape (kSplitShapes)
  bool colx = false;  // RMSNorm FP8 with a columnwise output: the single-pass band-exchange kernel
};

// rows longer than the row layouts (65536 elements) without an FP8 epilogue go to the split
// kernel (LayerNorm bf16 682 x 98304: 204 -> 79 us, RMSNorm 512 x 131072: 105 -> 63 us against
// the band kernel); up to 65536 the one-workgroup-per-row layout is faster (LayerNorm
// 1024 x 65536: 68 against 72 us; RMSNorm 52 against 63 us)
constexpr int64_t kSplitMinHidden = 65536 + 8;
// 16-bit input, the 8-wave shapes with gamma in registers (bf16, one box, against the default
// before them): LayerNorm from 32769 elements, 16384-column slices up to 49152 (2048 x 40960
// 84.6 against 96.3 us in the row layout, 1536 x 49152 69.2 against 73.8 on 32768-column
// slices, whose second slice would hold 16384 columns) and 32768-column slices beyond (1024 x
// 57344 58.5 against 63.5 on 16384 columns); RMSNorm from 65537, 16384-column slices up to
// 131072 (768 x 81920 54.8 against 59.8 us, 512 x 131072 57.6 against 62.3 on the 16-wave
// shape) and 32768-column slices beyond (256 x 262144 65.6 against 114.6 in the band kernel)
constexpr int64_t kSplitMinHiddenLn16 = 32768 + 1;
constexpr int64_t kSplitShape2MaxLn16 = 49152;
constexpr int64_t kSplitShape2MaxRms16 = 131072;

int plan_fwd(int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int out_dtype, int norm_type,
             int scaling, int qlayout, int cu_margin, FwdPlan *pl) {
  if (rows < 0 || hidden <= 0) return fail(NORM_ERR_INVALID_ARG, "rows must be >= 0 and hidden > 0");
  if (norm_type != NORM_LAYERNORM && norm_type != NORM_RMSNORM)
    return fail(NORM_ERR_INVALID_ARG, "unknown norm_type %d", norm_type);
  if (!is_hp(in_dtype)) return fail(NORM_ERR_UNSUPPORTED, "input dtype %d not supported", in_dtype);
  if (!is_hp(w_dtype)) return fail(NORM_ERR_UNSUPPORTED, "weight dtype %d not supported", w_dtype);
  if (cu_margin < 0) return fail(NORM_ERR_INVALID_ARG, "cu_margin must be >= 0");
  const bool scales_padded = (qlayout & NORM_Q_SCALES_PADDED) != 0;
  qlayout &= ~NORM_Q_SCALES_PADDED;
  const bool col_rowmajor = (qlayout & NORM_Q_COLWISE_ROWMAJOR) != 0;
  if (col_rowmajor) {
    if (!(qlayout & NORM_Q_COLWISE))
      return fail(NORM_ERR_INVALID_ARG, "NORM_Q_COLWISE_ROWMAJOR modifies a columnwise layout");
    qlayout &= ~NORM_Q_COLWISE_ROWMAJOR;
  }
  if (qlayout < NORM_Q_ROWWISE || qlayout > NORM_Q_ROWWISE_COLWISE)
    return fail(NORM_ERR_INVALID_ARG, "unknown quantize layout %d", qlayout);
  if (hidden > (int64_t)1 << 24) return fail(NORM_ERR_UNSUPPORTED, "hidden above 2^24 not supported");
  pl->gen = hidden % 8 != 0;
  switch (scaling) {
    case NORM_SCALING_NONE:
      if (!is_hp(out_dtype)) return fail(NORM_ERR_UNSUPPORTED, "no-scaling output must be F32/F16/BF16");
      if (qlayout != NORM_Q_ROWWISE) return fail(NORM_ERR_UNSUPPORTED, "no-scaling output is rowwise only");
      pl->mode = MODE_PLAIN;
      break;
    case NORM_SCALING_DELAYED_TENSOR:
    case NORM_SCALING_MXFP8_1D32:
    case NORM_SCALING_MXFP8_1D32_CEIL:
      if (!is_fp8(out_dtype)) return fail(NORM_ERR_UNSUPPORTED, "scaled output must be FP8_E4M3 or FP8_E5M2");
      pl->mode = scaling == NORM_SCALING_DELAYED_TENSOR ? MODE_DELAYED : MODE_MX;
      break;
    default:
      return fail(NORM_ERR_INVALID_ARG, "unknown scaling mode %d", scaling);
  }
  if (scales_padded && pl->mode != MODE_MX)
    return fail(NORM_ERR_INVALID_ARG, "NORM_Q_SCALES_PADDED applies to MXFP8 scaling only");
  pl->scales_padded = scales_padded;
  pl->rowwise = (qlayout & NORM_Q_ROWWISE) != 0;
  pl->colwise = (qlayout & NORM_Q_COLWISE) != 0;

  // layout choice
  const int force_band = knob(K_FORCE_BAND, 0);
  int row_cfg = -1;
  const int row_override = knob(K_ROW_CFG, -1);
  if (row_override >= 0 && row_override < ROW_NCFG && kRowShapes[row_override].cover() >= hidden) {
    row_cfg = row_override;
  } else {
    // (from a sweep over row lengths) LayerNorm stages twice the weights of RMSNorm in LDS: for
    // rows of 4097..8192 elements four rows share one copy (a 4-row workgroup), where one row
    // per workgroup would leave a CU with 8 waves; for 8193..16384 two rows of 8 waves share
    // 128 KB of LDS weights (16 waves per CU, where the weights in registers left room for 8:
    // bf16 16384 x 12288 192 -> 163 us); RMSNorm rows of 8193..16384 elements run on 16 waves
    // with their few weights in registers, two workgroups per CU
    const int pref_ln[] = {ROW_W1_K1,   ROW_W1_K2,   ROW_W1_K4,  ROW_W2T2_K4,
                           ROW_W4T4_K4, ROW_W8T2_K4, ROW_W16_K4, ROW_W16_K8};
    const int pref_rms[] = {ROW_W1_K1, ROW_W1_K2,  ROW_W1_K4,  ROW_W2T2_K4,
                            ROW_W4_K4, ROW_W16_K2, ROW_W16_K4, ROW_W16_K8};
    for (int c : norm_type == NORM_LAYERNORM ? pref_ln : pref_rms)
      if (kRowShapes[c].cover() >= hidden) {
        row_cfg = c;
        break;
      }
    // RMSNorm rows of 4097..8192 elements with an FP8 epilogue (1-byte codes): four rows per
    // workgroup (delayed E4M3 32768 x 8192: 146 -> 138 us; MXFP8 143 -> 137 us); with a 2-byte
    // output one row per workgroup stays faster at 8192 (187 against 205 us)
    if (norm_type == NORM_RMSNORM && row_cfg == ROW_W4_K4 && pl->mode != MODE_PLAIN) row_cfg = ROW_W4T4_K4;
    // LayerNorm rows of 16385..32768 elements, 16-bit input, no FP8 epilogue: 8 waves with gamma
    // and beta in registers and the next row prefetched, where 16 waves must read the weights
    // from the caches per strip (bf16 2048 x 32768: 76 -> 54 us; 4096 x 16392: 105 -> 69 us)
    if (norm_type == NORM_LAYERNORM && row_cfg == ROW_W16_K4 && pl->mode == MODE_PLAIN && in_dtype != DT_F32)
      row_cfg = ROW_W8_K8;
    // and rows of 8193..16384: 4 waves with gamma and beta in registers, where the two rows of 8
    // waves sharing 128 KB of LDS weights read those 128 KB from LDS for every row (bf16 16384 x
    // 12288: 163-168 -> 149 us; 19660 x 10240: 184-189 -> 152 us; 12288 x 16384: 152 -> 143.5 us)
    if (norm_type == NORM_LAYERNORM && row_cfg == ROW_W8T2_K4 && pl->mode == MODE_PLAIN && in_dtype != DT_F32)
      row_cfg = ROW_W4_K8;
  }
  // a columnwise output goes through the statistics pass + tile kernel when a row layout covers
  // the row (NORMFP8_COL_KERNEL=0 selects the single-pass band kernel instead)
  // (the tile kernel's lane offsets are 32-bit: 128 rows of float32 input, 128 columns of the
  // transposed output)
  const bool tile_fits = (int64_t)hidden * 4 * kColTileRows < (1ll << 32) && rows * kColTileCols < (1ll << 32);
  pl->col = pl->colwise && row_cfg >= 0 && tile_fits && !force_band && knob(K_COL_KERNEL, 1) != 0;
  pl->band = !pl->col && (pl->colwise || row_cfg < 0 || force_band);
  pl->col_rowmajor = col_rowmajor;
  // delayed scaling with both outputs: the columnwise codes are the rowwise codes transposed
  // (one scale for the whole tensor), so the row kernel writes the rowwise codes and a byte
  // transpose reads them back, instead of a statistics pass and a second read of x
  pl->tr = pl->col && pl->mode == MODE_DELAYED && pl->rowwise && !col_rowmajor && hidden % 16 == 0 &&
           knob(K_DELAYED_TRANSPOSE, 1) != 0;
  // RMSNorm FP8 rowwise outputs: rows of 8193..16384 elements on 8 waves x 4 strips (16384 x
  // 12288: delayed 126 -> 113 us, MXFP8 130 -> 111 us; x 10240: 132 -> 111, 122 -> 101 us;
  // equal at 16384), rows of 2049..4096 on 4 waves x 2 rows x 2 strips (16384 x 4096: delayed
  // 43-45 -> 39 us, MXFP8 39 -> 36.5 us); with a 2-byte output the defaults stay faster. A
  // columnwise request keeps the default layout: its transpose route and its statistics + tile
  // route then reduce every row in the same order and give the same bytes.
  if (norm_type == NORM_RMSNORM && row_override < 0 && pl->mode != MODE_PLAIN && !pl->col) {
    if (row_cfg == ROW_W16_K2) row_cfg = ROW_W8_K4;
    else if (row_cfg == ROW_W2T2_K4) row_cfg = ROW_W4T2_K2;
  }
  if (pl->gen) {  // the general kernels: rows, then (columnwise) the column pass
    pl->col = pl->band = false;
  } else if (col_rowmajor && !pl->col) {
    return fail(NORM_ERR_UNSUPPORTED, "the row-major columnwise layout needs rows a row layout covers "
                                      "(hidden <= 65536) and the tile path");
  }
  if (pl->gen) {
    // no layout to choose
  } else if (!pl->band) {
    pl->cfg = row_cfg;
  } else {
    int bc;
    if (pl->colwise) bc = hidden <= 512 ? BAND_R8_K1 : BAND_R8_K2;
    else bc = hidden <= 2048 ? BAND_R1_K4 : BAND_R2_K8;
    const int band_override = knob(K_BAND_CFG, -1);
    if (band_override >= 0 && band_override < BAND_NCFG &&
        (kBandShapes[band_override].colwise_ok || !pl->colwise) &&
        !(pl->colwise && pl->mode == MODE_MX && kBandShapes[band_override].RW != 8))
      bc = band_override;
    pl->cfg = bc;
    pl->tile_rows = kBandShapes[bc].rows();
    pl->S = (int)cdiv(hidden, kBandShapes[bc].cols());
    pl->bands = cdiv(rows, pl->tile_rows);
    if (pl->S > kMaxSlices) {
      // more slices than a band can merge (columnwise output of rows beyond 64 K elements):
      // the general kernels, a row pass and a column pass
      if (col_rowmajor)
        return fail(NORM_ERR_UNSUPPORTED, "the row-major columnwise layout needs hidden <= 65536");
      pl->gen = true;
      pl->band = false;
      pl->S = 1;
    }
  }

  // long rows without an FP8 epilogue: the split kernel (NORMFP8_SPLIT=0 keeps the row / band
  // layouts, =1 takes the split kernel for any row it covers; NORMFP8_SPLIT_SHAPE=0 / 1 / 2 picks
  // its shape)
  {
    const int force = knob(K_SPLIT, -1);
    // shapes 1 and 2 (8 waves, gamma in registers) take 16-bit input only: the shape whose slices
    // divide the row more evenly (a short last slice idles its workgroups for most of a row)
    const bool in16 = in_dtype != DT_F32;
    const bool ln = norm_type == NORM_LAYERNORM;
    const int shape_ov = knob(K_SPLIT_SHAPE, -1);
    int shape = 0;
    if (in16) shape = hidden <= (ln ? kSplitShape2MaxLn16 : kSplitShape2MaxRms16) ? 2 : 1;
    if (shape_ov == 0) shape = 0;
    else if ((shape_ov == 1 || shape_ov == 2) && in16) shape = shape_ov;
    const int64_t min_hidden = in16 && ln ? kSplitMinHiddenLn16 : kSplitMinHidden;
    const int64_t S = cdiv(hidden, kSplitShapes[shape].cols());
    const bool fits = pl->mode == MODE_PLAIN && !pl->colwise && !pl->gen && !force_band && S <= kSplitMaxSlices;
    if (fits && (force == 1 || (force < 0 && hidden >= min_hidden))) {
      pl->split = true;
      pl->split_shape = shape;
      pl->band = pl->col = false;
      pl->S = (int)S;
    }
  }

  // RMSNorm FP8 with a transposed columnwise output, hidden a multiple of 512 and rows a
  // multiple of 128: one pass over x, the bands' row sums exchanged between the slices
  // (NORMFP8_COLX=0 keeps the two-pass routes)
  // (float32 input keeps the two-pass routes: two bands of it would fill the registers)
  if (norm_type == NORM_RMSNORM && pl->colwise && !col_rowmajor && !pl->gen && pl->mode != MODE_PLAIN &&
      in_dtype != DT_F32 &&
      hidden % kColxCols == 0 && rows > 0 && rows % kColxRows == 0 && rows * (int64_t)kColxRows < (1ll << 32) &&
      (int64_t)kColxRows * hidden * 2 < (1ll << 32) &&
      knob(K_COLX, 1) != 0) {
    pl->colx = true;
    pl->S = (int)(hidden / kColxCols);
  }

  // workspace: header when the launch coordinates workgroups, then band or split partials
  const bool header = pl->mode == MODE_DELAYED || (pl->band && pl->S > 1) || pl->split || pl->colx;
  if (pl->gen) pl->cfg = 0;
  size_t ws = header ? (size_t)kWsHeaderBytes : 0;
  if (pl->band && pl->S > 1) {
    pl->partial_off = ws;
    const int nv = norm_type == NORM_LAYERNORM ? 3 : 1;  // (mean, M2, shift) or the sum of squares
    ws += round_up((size_t)pl->bands * pl->S * pl->tile_rows * nv * sizeof(uint64_t), 256);
  }
  if (pl->split) {
    pl->partial_off = ws;
    const int nv = norm_type == NORM_LAYERNORM ? 3 : 1;
    ws += round_up((size_t)rows * pl->S * nv * sizeof(uint64_t), 256);
  }
  if (pl->colx) {
    pl->colx_off = ws;
    ws += round_up((size_t)rows * pl->S * sizeof(uint64_t), 256);
  }
  // row statistics of a columnwise request (two-pass paths; sized for every columnwise request,
  // since unaligned tensors send any request to the general kernels at launch)
  if (pl->colwise) {
    pl->stats_off = ws;
    ws += round_up((size_t)rows * sizeof(float) * (norm_type == NORM_LAYERNORM ? 2 : 1), 256);
  }
  pl->ws_bytes = ws;
  (void)in_dtype;
  (void)w_dtype;
  return NORM_OK;
}

// ---------------------------------------------------------------- backward plan
struct BwdPlan {
  int cfg = 0;
  int64_t G_max = 0;  // partial rows the workspace holds
  size_t ws_bytes = 0;
  bool gen = false;   // general kernels (hidden not a multiple of 8, or beyond the row layouts)
};
constexpr int kGenChunks = 256;  // most row chunks (weight-gradient partials) of the general backward

constexpr int kMaxCus = 256;  // gfx950 (MI355X) compute units; bounds the workspace query

int bwd_wgs_per_cu(int cfg) {
  const int w = kBwdShapes[cfg].W * kBwdShapes[cfg].T;
  return w >= 8 ? 1 : 8 / w;
}

int plan_bwd(int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int norm_type, int cu_margin,
             BwdPlan *pl) {
  if (rows < 0 || hidden <= 0) return fail(NORM_ERR_INVALID_ARG, "rows must be >= 0 and hidden > 0");
  if (norm_type != NORM_LAYERNORM && norm_type != NORM_RMSNORM)
    return fail(NORM_ERR_INVALID_ARG, "unknown norm_type %d", norm_type);
  if (!is_hp(in_dtype)) return fail(NORM_ERR_UNSUPPORTED, "input dtype %d not supported", in_dtype);
  if (!is_hp(w_dtype)) return fail(NORM_ERR_UNSUPPORTED, "weight dtype %d not supported", w_dtype);
  if (cu_margin < 0) return fail(NORM_ERR_INVALID_ARG, "cu_margin must be >= 0");
  if (hidden > (int64_t)1 << 24) return fail(NORM_ERR_UNSUPPORTED, "hidden above 2^24 not supported");
  int cfg = -1;
  const int ov = knob(K_BWD_CFG, -1);
  if (ov >= 0 && ov < BWD_NCFG && kBwdShapes[ov].cover() >= hidden) {
    cfg = ov;
  } else {
    const int pref[] = {BWD_W2_K1, BWD_W4_K1, BWD_W4_K2, BWD_W5_K2_T2, BWD_W8_K2, BWD_W8_K3, BWD_W16_K2};
    for (int c : pref)
      if (kBwdShapes[c].cover() >= hidden) {
        cfg = c;
        break;
      }
  }
  const int arrays = norm_type == NORM_LAYERNORM ? 2 : 1;
  if (cfg < 0 || hidden % 8 != 0) {  // the general kernels
    pl->gen = true;
    pl->cfg = -1;
    pl->G_max = kGenChunks;
    pl->ws_bytes = kWsHeaderBytes + round_up((size_t)pl->G_max * round_up((size_t)hidden, 32) * arrays * sizeof(float), 256);
    return NORM_OK;
  }
  // with few rows per team (under four), one-team workgroups: the merge of the teams' partial
  // sums would cost more than the smaller partial traffic saves
  if (ov < 0 && rows < (int64_t)kMaxCus * kBwdShapes[cfg].T * 4) {
    if (cfg == BWD_W2_K1) cfg = BWD_W2_K1_T1;
    else if (cfg == BWD_W4_K1) cfg = BWD_W4_K1_T1;
    else if (cfg == BWD_W4_K2) cfg = BWD_W4_K2_T1;
    else if (cfg == BWD_W5_K2_T2) cfg = BWD_W5_K2_T1;
  }
  pl->cfg = cfg;
  const int64_t gmax = (int64_t)kMaxCus * bwd_wgs_per_cu(cfg);
  pl->G_max = rows < gmax ? (rows > 0 ? rows : 1) : gmax;
  // (a launch with unaligned tensors takes the general kernels, whose partials fit as well)
  if (pl->G_max < kGenChunks) pl->G_max = kGenChunks;
  pl->ws_bytes = kWsHeaderBytes + round_up((size_t)pl->G_max * round_up((size_t)hidden, 32) * arrays * sizeof(float), 256);
  return NORM_OK;
}

// Persistent grid of the backward row kernel: one workgroup per CU (more for small layouts),
// capped by the workspace's partial rows and by the row count in units of the layout's T teams,
// so that every workgroup's first base row b * T is a row of the tensor.
int64_t bwd_grid(const BwdPlan &pl, int cus_free, int occ, int64_t rows) {
  const int per_cu = bwd_wgs_per_cu(pl.cfg);
  int64_t G = (int64_t)cus_free * (occ < per_cu ? occ : per_cu);
  if (G > pl.G_max) G = pl.G_max;
  const int64_t slots = cdiv(rows, kBwdShapes[pl.cfg].T);
  if (G > slots) G = slots;
  if (G < 1) G = 1;
  return G;
}

bool aligned_to(const void *p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
size_t elem_bytes(int dt) { return dt == DT_F32 ? 4 : (is_hp(dt) ? 2 : 1); }

int check_ws(void *ws, size_t have, size_t need) {
  if (need == 0) return NORM_OK;
  if (!ws) return fail(NORM_ERR_INVALID_ARG, "workspace is NULL but %zu bytes are required", need);
  if (!aligned16(ws)) return fail(NORM_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (have < need) return fail(NORM_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", have, need);
  return NORM_OK;
}

}  // namespace

namespace nf8 {
int set_last_error(int code, const char *msg) { return fail(code, "%s", msg); }
}  // namespace nf8

// ================================================================ C ABI
extern "C" {

int norm_abi_version(void) { return NORMFP8_ABI_VERSION; }

const char *norm_last_error(void) { return g_err.c_str(); }

int norm_fwd_workspace_size(int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int out_dtype,
                            int norm_type, int scaling, int qlayout, int zero_centered_gamma,
                            float epsilon, int cu_margin, int is_training, size_t *bytes) {
  (void)zero_centered_gamma;
  (void)epsilon;
  (void)is_training;
  if (!bytes) return fail(NORM_ERR_INVALID_ARG, "bytes is NULL");
  FwdPlan pl;
  int rc = plan_fwd(rows, hidden, in_dtype, w_dtype, out_dtype, norm_type, scaling, qlayout, cu_margin, &pl);
  if (rc) return rc;
  *bytes = pl.ws_bytes;
  return ok();
}

int norm_bwd_workspace_size(int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int norm_type,
                            int zero_centered_gamma, float epsilon, int cu_margin, int with_add,
                            size_t *bytes) {
  (void)zero_centered_gamma;
  (void)epsilon;
  if (!bytes) return fail(NORM_ERR_INVALID_ARG, "bytes is NULL");
  if (with_add && norm_type != NORM_RMSNORM)
    return fail(NORM_ERR_INVALID_ARG, "the fused backward-add is defined for RMSNorm only");
  BwdPlan pl;
  int rc = plan_bwd(rows, hidden, in_dtype, w_dtype, norm_type, cu_margin, &pl);
  if (rc) return rc;
  *bytes = pl.ws_bytes;
  return ok();
}

int norm_fwd(void *stream, const void *x, const void *gamma, const void *beta, const float *scale,
             const float *amax, void *y, void *y_colwise, float *mu, float *rsigma, void *scale_inv,
             void *colwise_scale_inv, float *updated_amax, void *workspace, size_t workspace_bytes,
             int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int out_dtype, int norm_type,
             int scaling, int qlayout, int zero_centered_gamma, float epsilon, int cu_margin) {
  FwdPlan pl;
  int rc = plan_fwd(rows, hidden, in_dtype, w_dtype, out_dtype, norm_type, scaling, qlayout, cu_margin, &pl);
  if (rc) return rc;
  const bool ln = norm_type == NORM_LAYERNORM;
  const bool any = rows > 0;  // with no rows, row-indexed buffers may be NULL
  if ((any && !x) || !gamma) return fail(NORM_ERR_INVALID_ARG, "x and gamma are required");
  if (ln && !beta) return fail(NORM_ERR_INVALID_ARG, "beta is required for LayerNorm");
  if (!ln && beta) return fail(NORM_ERR_INVALID_ARG, "beta must be NULL for RMSNorm");
  if (any && pl.rowwise && !y) return fail(NORM_ERR_INVALID_ARG, "rowwise output y is NULL");
  if (!pl.rowwise && y) return fail(NORM_ERR_INVALID_ARG, "y must be NULL when rowwise output is not requested");
  if (any && pl.colwise && !y_colwise) return fail(NORM_ERR_INVALID_ARG, "columnwise output y_colwise is NULL");
  if (!pl.colwise && y_colwise) return fail(NORM_ERR_INVALID_ARG, "y_colwise must be NULL for a rowwise-only layout");
  if (pl.mode == MODE_DELAYED) {
    if (!scale || !amax || !updated_amax)
      return fail(NORM_ERR_INVALID_ARG, "delayed scaling needs scale, amax and updated_amax");
  }
  if (pl.mode == MODE_DELAYED || (pl.mode == MODE_MX && any)) {
    if (pl.rowwise && !scale_inv) return fail(NORM_ERR_INVALID_ARG, "scale_inv is required for rowwise output");
    if (pl.colwise && !colwise_scale_inv)
      return fail(NORM_ERR_INVALID_ARG, "colwise_scale_inv is required for columnwise output");
  }
  if (!(epsilon >= 0.0f)) return fail(NORM_ERR_INVALID_ARG, "epsilon must be >= 0");
  // tensors must be aligned to their element size; the vector kernels need 16 bytes, anything
  // less goes to the general kernels
  {
    const void *ptrs[] = {x, gamma, beta, y, y_colwise, mu, rsigma};
    const size_t sizes[] = {elem_bytes(in_dtype), elem_bytes(w_dtype), elem_bytes(w_dtype), elem_bytes(out_dtype),
                            1, 4, 4};
    for (int i = 0; i < 7; ++i) {
      if (!ptrs[i]) continue;
      if (!aligned_to(ptrs[i], sizes[i]))
        return fail(NORM_ERR_MISALIGNED, "tensor pointers must be aligned to their element size");
      if (i < 5 && !aligned16(ptrs[i])) pl.gen = true;
    }
    if (pl.mode == MODE_DELAYED)
      for (const void *q : {(const void *)scale, (const void *)amax, (const void *)updated_amax, (const void *)scale_inv,
                            (const void *)colwise_scale_inv})
        if (q && !aligned_to(q, 4)) return fail(NORM_ERR_MISALIGNED, "float32 scalars must be 4-byte aligned");
  }
  rc = check_ws(workspace, workspace_bytes, pl.ws_bytes);
  if (rc) return rc;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rows == 0) {
    if (pl.mode != MODE_DELAYED) return ok();  // nothing to compute
    // delayed scaling still publishes updated_amax = amax and scale_inv = 1/scale: one
    // workgroup of the (general) row kernel does that without visiting any row
    pl.band = false;
    pl.col = false;
    pl.gen = true;
  }

  DeviceInfo dev;
  rc = device_info(&dev);
  if (rc) return rc;
  if (cu_margin >= dev.cus) return fail(NORM_ERR_INVALID_ARG, "cu_margin (%d) >= CU count (%d)", cu_margin, dev.cus);

  FwdRowParams f{};
  f.x = x;
  f.gamma = gamma;
  f.beta = beta;
  f.scale = scale;
  f.amax_in = amax;
  f.y = y;
  f.mu = ln ? mu : nullptr;
  f.rsigma = rsigma;
  f.scale_inv = scale_inv;
  f.updated_amax = updated_amax;
  f.ws = static_cast<uint32_t *>(workspace);
  f.rows = rows;
  f.hidden = hidden;
  // E8M0 grid row strides (padded: the block-count dimension to a multiple of 4, the other
  // dimension, which only the allocation sees, to a multiple of 128)
  f.mx_cols = pl.scales_padded ? (int64_t)round_up((size_t)cdiv(hidden, 32), 4) : cdiv(hidden, 32);
  const int64_t col_ld = pl.col_rowmajor ? (pl.scales_padded ? (int64_t)round_up((size_t)hidden, 128) : hidden)
                                         : (pl.scales_padded ? (int64_t)round_up((size_t)cdiv(rows, 32), 4)
                                                             : cdiv(rows, 32));
  f.w_dtype = w_dtype;
  f.out_dtype = out_dtype;
  f.mx_ceil = scaling == NORM_SCALING_MXFP8_1D32_CEIL ? 1 : 0;
  f.zero_centered = zero_centered_gamma ? 1 : 0;
  f.eps = epsilon;

  auto launch_rows = [&](const FwdRowParams &rp, int mode) -> int {
    const void *fn = fwd_row_kernel_ptr(norm_type, in_dtype, mode, pl.cfg);
    if (!fn) return fail(NORM_ERR_UNSUPPORTED, "no forward row kernel for this combination");
    const RowShape &sh = kRowShapes[pl.cfg];
    int occ = 1;
    int r = occupancy(fn, sh.threads(), &occ);
    if (r) return r;
    const int occ_cap = knob(K_ROW_OCC, 0);  // tuning: fewer workgroups per CU
    if (occ_cap > 0 && occ_cap < occ) occ = occ_cap;
    const int64_t slots = cdiv(rows, sh.T);
    int64_t cap = (int64_t)(dev.cus - cu_margin) * occ;
    if (cap > kMaxGrid) cap = kMaxGrid;
    // persistent grid: as many workgroups as give every one the same number of rows, so that
    // the last round does not run on a fraction of the grid
    const int64_t rounds = cdiv(slots, cap < 1 ? 1 : cap);
    int64_t grid = cdiv(slots, rounds < 1 ? 1 : rounds);
    if (knob(K_ROW_BALANCE, 1) == 0) grid = slots < cap ? slots : cap;
    if (grid < 1) grid = 1;
    FwdRowParams copy = rp;
    return launch(fn, dim3((unsigned)grid), dim3(sh.threads()), &copy, st);
  };
  if (pl.gen) {
    // rows (statistics and rowwise output; delayed scaling's amax), then the column pass
    float *st_mu = nullptr, *st_rs = rsigma;
    if (pl.colwise) {
      if (!st_rs) st_rs = reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.stats_off);
      if (ln) st_mu = mu ? mu : reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.stats_off) + rows;
    }
    FwdRowParams r = f;
    r.mu = ln ? (pl.colwise ? st_mu : mu) : nullptr;
    r.rsigma = st_rs;
    int mode1 = pl.mode;
    if (!pl.rowwise) {
      r.y = nullptr;
      r.scale_inv = nullptr;
      if (mode1 == MODE_MX) mode1 = MODE_STATS;
    }
    const void *fn = fwd_gen_row_kernel_ptr(norm_type, in_dtype, mode1);
    if (!fn) return fail(NORM_ERR_UNSUPPORTED, "no general forward kernel for this combination");
    int occ = 1;
    rc = occupancy(fn, 256, &occ);
    if (rc) return rc;
    int64_t grid = cdiv(rows, 4);
    int64_t cap = (int64_t)(dev.cus - cu_margin) * occ;
    if (cap > kMaxGrid) cap = kMaxGrid;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    rc = launch(fn, dim3((unsigned)grid), dim3(256), &r, st);
    if (rc) return rc;
    if (pl.colwise && (rows > 0 || pl.mode == MODE_DELAYED)) {  // (delayed: colwise_scale_inv too)
      FwdTileParams tp{};
      tp.f = f;
      tp.y_col = y_colwise;
      tp.col_scale_inv = colwise_scale_inv;
      tp.st_mu = st_mu;
      tp.st_rs = st_rs;
      tp.mx_rows = cdiv(rows, 32);
      tp.mx_col_ld = col_ld;
      tp.col_rowmajor = pl.col_rowmajor ? 1 : 0;
      const void *fc = fwd_gen_col_kernel_ptr(norm_type, in_dtype, pl.mode, pl.col_rowmajor);
      if (!fc) return fail(NORM_ERR_UNSUPPORTED, "no general columnwise kernel for this combination");
      const int64_t items = cdiv(hidden, 64) * tp.mx_rows;
      const int64_t g2 = items < 1 ? 1 : (items < (1 << 20) ? items : (1 << 20));
      rc = launch(fc, dim3((unsigned)g2), dim3(64), &tp, st);
      if (rc) return rc;
    }
    return ok();
  }
  if (pl.split) {
    const void *fn = fwd_split_kernel_ptr(norm_type, in_dtype, pl.split_shape);
    if (!fn) return fail(NORM_ERR_UNSUPPORTED, "no split kernel for this combination");
    const int split_threads = kSplitShapes[pl.split_shape].threads;
    int occ = 1;
    rc = occupancy(fn, split_threads, &occ);
    if (rc) return rc;
    int64_t cap = (int64_t)(dev.cus - cu_margin) * occ;
    if (cap > kMaxGrid) cap = kMaxGrid;
    int64_t groups = cap / pl.S;
    if (groups > rows) groups = rows;
    if (groups < 1)
      return fail(NORM_ERR_UNSUPPORTED, "cu_margin %d leaves fewer than the %d resident workgroups a split row needs",
                  cu_margin, pl.S);
    FwdSplitParams sp{};
    sp.f = f;
    sp.partials = reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) + pl.partial_off);
    sp.S = pl.S;
    rc = launch(fn, dim3((unsigned)(groups * pl.S)), dim3(split_threads), &sp, st);
    if (rc) return rc;
    return ok();
  }
  if (pl.colx) {
    // (the two-pass routes serve what this kernel cannot: scale grids not 16 / 4-byte aligned, or
    // a CU margin that leaves fewer resident workgroups than one band's slices)
    const void *fn = fwd_colx_kernel_ptr(in_dtype, out_dtype, pl.mode);
    int occ = 1;
    if (fn) {
      rc = occupancy(fn, kColxThreads, &occ);
      if (rc) return rc;
    }
    int64_t cap = (int64_t)(dev.cus - cu_margin) * occ;
    if (cap > kMaxGrid) cap = kMaxGrid;
    int64_t groups = cap / pl.S;
    const int64_t nbands = rows / kColxRows;
    if (groups > nbands) groups = nbands;
    const bool scales_ok = pl.mode != MODE_MX || ((!pl.rowwise || aligned16(scale_inv)) && aligned_to(colwise_scale_inv, 4));
    if (fn && groups >= 1 && scales_ok) {
      FwdColxParams cp{};
      cp.f = f;
      cp.y_col = y_colwise;
      cp.col_scale_inv = colwise_scale_inv;
      cp.partials = reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) + pl.colx_off);
      cp.mx_col_ld = col_ld;
      cp.S = pl.S;
      cp.write_row = pl.rowwise ? 1 : 0;
      if (!pl.rowwise) cp.f.y = nullptr;
      rc = launch(fn, dim3((unsigned)(groups * pl.S)), dim3(kColxThreads), &cp, st);
      if (rc) return rc;
      return ok();
    }
    // otherwise the route planned without it
  }
  if (!pl.band && !pl.col) {
    rc = launch_rows(f, pl.mode);
    if (rc) return rc;
    return ok();
  }
  if (pl.tr) {
    // rowwise codes, amax, scale_inv and the statistics; then the columnwise codes by transpose
    rc = launch_rows(f, MODE_DELAYED);
    if (rc) return rc;
    TransposeParams t{};
    t.src = static_cast<const uint8_t *>(y);
    t.dst = static_cast<uint8_t *>(y_colwise);
    t.scale = scale;
    t.col_scale_inv = static_cast<float *>(colwise_scale_inv);
    t.rows = rows;
    t.hidden = hidden;
    // tile shape: 512 rows x 128 columns (512-byte column pieces; at 32768 x 8192 the call takes
    // 260 us against 265 us with 256 x 256 tiles and 279 us with 128 x 256)
    const int tc = knob(K_TRANSPOSE_TC, 128) == 256 ? 256 : 128;
    const int rl = tc == 128 || knob(K_TRANSPOSE_RL, 8) != 4 ? 8 : 4;
    t.tiles_r = cdiv(rows, tc == 128 ? 512 : 32 * rl);
    t.tiles_c = cdiv(hidden, tc);
    const void *fn = transpose_u8_kernel_ptr(rl, tc);
    if (!fn) return fail(NORM_ERR_UNSUPPORTED, "no transpose kernel for this tile shape");
    int occ = 1;
    rc = occupancy(fn, kTrThreads, &occ);
    if (rc) return rc;
    int64_t cap = (int64_t)(dev.cus - cu_margin) * occ;
    if (cap > kMaxGrid) cap = kMaxGrid;
    const int64_t tiles = t.tiles_r * t.tiles_c;
    const int64_t grid = tiles < cap ? tiles : cap;
    rc = launch(fn, dim3((unsigned)(grid < 1 ? 1 : grid)), dim3(kTrThreads), &t, st);
    if (rc) return rc;
    return ok();
  }
  if (pl.col) {
    // pass 1: statistics of every row, into the caller's mu / rsigma or the workspace
    float *st_mu = nullptr;
    float *st_rs = rsigma ? rsigma : reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.stats_off);
    if (ln) st_mu = mu ? mu : reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.stats_off) + rows;
    FwdRowParams s = f;
    s.y = nullptr;
    s.mu = st_mu;
    s.rsigma = st_rs;
    rc = launch_rows(s, MODE_STATS);
    if (rc) return rc;
    // pass 2: independent 128 x 128 tiles
    FwdTileParams tp{};
    tp.f = f;
    tp.y_col = y_colwise;
    tp.col_scale_inv = colwise_scale_inv;
    tp.st_mu = st_mu;
    tp.st_rs = st_rs;
    tp.mx_rows = cdiv(rows, 32);
    tp.mx_col_ld = col_ld;
    tp.tiles_r = cdiv(rows, kColTileRows);
    tp.tiles_c = cdiv(hidden, kColTileCols);
    tp.write_row = pl.rowwise ? 1 : 0;
    tp.col_rowmajor = pl.col_rowmajor ? 1 : 0;
    const void *fn = fwd_tile_kernel_ptr(norm_type, in_dtype, pl.mode, pl.col_rowmajor);
    if (!fn) return fail(NORM_ERR_UNSUPPORTED, "no forward tile kernel for this combination");
    int occ = 1;
    rc = occupancy(fn, kColThreads, &occ);
    if (rc) return rc;
    int64_t cap = (int64_t)(dev.cus - cu_margin) * occ;
    if (cap > kMaxGrid) cap = kMaxGrid;
    const int64_t tiles = tp.tiles_r * tp.tiles_c;
    const int64_t grid = tiles < cap ? tiles : cap;
    rc = launch(fn, dim3((unsigned)grid), dim3(kColThreads), &tp, st);
    if (rc) return rc;
    return ok();
  }

  FwdBandParams b{};
  b.f = f;
  b.y_col = y_colwise;
  b.col_scale_inv = colwise_scale_inv;
  b.partials = pl.S > 1 ? reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) + pl.partial_off) : nullptr;
  b.bands = pl.bands;
  b.mx_rows = cdiv(rows, 32);
  b.mx_col_ld = col_ld;
  b.S = pl.S;
  b.write_row = pl.rowwise ? 1 : 0;
  const void *fn = fwd_band_kernel_ptr(norm_type, in_dtype, pl.mode, pl.colwise, pl.cfg);
  if (!fn) return fail(NORM_ERR_UNSUPPORTED, "no forward band kernel for this combination");
  const int threads = 256;
  // persistent grid: at most what fits on the CUs left by the margin; the S workgroups of a
  // band wait for each other, so at least S must be able to run at once
  int occ = 1;
  rc = occupancy(fn, threads, &occ);
  if (rc) return rc;
  int64_t cap = (int64_t)(dev.cus - cu_margin) * occ;
  if (cap > kMaxGrid) cap = kMaxGrid;
  if (pl.S > 1 && cap < 2 * pl.S)
    return fail(NORM_ERR_UNSUPPORTED, "cu_margin %d leaves too few resident workgroups for %d slices", cu_margin,
                pl.S);
  const int64_t tiles = pl.bands * pl.S;
  int64_t grid = tiles < cap ? tiles : cap;
  // ticket classes: one per XCD when every class gets several bands and at least 2S workgroups
  b.classes = 1;
  if (grid >= (int64_t)kClasses * 2 * pl.S && pl.bands >= (int64_t)kClasses * 4 &&
      knob(K_BAND_CLASSES, kClasses) == kClasses) {
    b.classes = kClasses;
    grid = grid / kClasses * kClasses;
  }
  rc = launch(fn, dim3((unsigned)grid), dim3(threads), &b, st);
  if (rc) return rc;
  return ok();
}

static int bwd_common(void *stream, bool with_add, const void *dy, const void *x, const void *residual, const float *mu,
                      const float *rsigma, const void *gamma, void *dx, void *dgamma, void *dbeta,
                      void *workspace, size_t workspace_bytes, int64_t rows, int64_t hidden, int in_dtype,
                      int w_dtype, int norm_type, int zero_centered_gamma, int cu_margin) {
  BwdPlan pl;
  int rc = plan_bwd(rows, hidden, in_dtype, w_dtype, norm_type, cu_margin, &pl);
  if (rc) return rc;
  const bool ln = norm_type == NORM_LAYERNORM;
  const bool any = rows > 0;  // with no rows, row-indexed buffers may be NULL
  if ((any && (!dy || !x || !rsigma || !dx)) || !gamma || !dgamma)
    return fail(NORM_ERR_INVALID_ARG, "dy, x, rsigma, gamma, dx and dgamma are required");
  if (ln && ((any && !mu) || !dbeta)) return fail(NORM_ERR_INVALID_ARG, "LayerNorm backward needs mu and dbeta");
  if (!ln && dbeta) return fail(NORM_ERR_INVALID_ARG, "dbeta must be NULL for RMSNorm");
  {
    const void *ptrs[] = {dy, x, residual, dx, gamma, dgamma, dbeta, mu, rsigma};
    const size_t sizes[] = {elem_bytes(in_dtype), elem_bytes(in_dtype), elem_bytes(in_dtype), elem_bytes(in_dtype),
                            elem_bytes(w_dtype), elem_bytes(w_dtype), elem_bytes(w_dtype), 4, 4};
    for (int i = 0; i < 9; ++i) {
      if (!ptrs[i]) continue;
      if (!aligned_to(ptrs[i], sizes[i]))
        return fail(NORM_ERR_MISALIGNED, "tensor pointers must be aligned to their element size");
      if (i < 5 && !aligned16(ptrs[i])) pl.gen = true;  // the vector kernels need 16 bytes
    }
  }
  rc = check_ws(workspace, workspace_bytes, pl.ws_bytes);
  if (rc) return rc;

  DeviceInfo dev;
  rc = device_info(&dev);
  if (rc) return rc;
  if (cu_margin >= dev.cus) return fail(NORM_ERR_INVALID_ARG, "cu_margin (%d) >= CU count (%d)", cu_margin, dev.cus);
  hipStream_t st = static_cast<hipStream_t>(stream);

  if (pl.gen) {
    // dx one wave per row, then the weight-gradient partials of row chunks, then the finalize
    BwdParams p{};
    p.dy = dy;
    p.x = x;
    p.residual = residual;
    p.mu = ln ? mu : nullptr;
    p.rsigma = rsigma;
    p.gamma = gamma;
    p.dx = dx;
    p.part = reinterpret_cast<float *>(static_cast<char *>(workspace) + kWsHeaderBytes);
    p.rows = rows;
    p.hidden = hidden;
    p.w_dtype = w_dtype;
    p.zero_centered = zero_centered_gamma ? 1 : 0;
    int64_t G = rows / 16;
    if (G > kGenChunks) G = kGenChunks;
    if (G < 1) G = 1;
    p.G = (int)G;
    if (rows > 0) {
      const void *fr = bwd_gen_row_kernel_ptr(norm_type, in_dtype, with_add);
      if (!fr) return fail(NORM_ERR_UNSUPPORTED, "no general backward kernel for this combination");
      int occ = 1;
      rc = occupancy(fr, 256, &occ);
      if (rc) return rc;
      int64_t grid = cdiv(rows, 4);
      const int64_t cap = (int64_t)(dev.cus - cu_margin) * occ;
      if (grid > cap) grid = cap;
      if (grid < 1) grid = 1;
      rc = launch(fr, dim3((unsigned)grid), dim3(256), &p, st);
      if (rc) return rc;
    }
    const void *fw = bwd_gen_wgrad_kernel_ptr(norm_type, in_dtype);
    if (!fw) return fail(NORM_ERR_UNSUPPORTED, "no general weight-gradient kernel for this combination");
    const int64_t items = cdiv(hidden, 64) * G;
    rc = launch(fw, dim3((unsigned)(items < (1 << 20) ? items : (1 << 20))), dim3(64), &p, st);
    if (rc) return rc;
    FinalizeParams fp{};
    fp.part = p.part;
    fp.dgamma = dgamma;
    fp.dbeta = ln ? dbeta : nullptr;
    fp.hidden = hidden;
    fp.G = (int)G;
    fp.w_dtype = w_dtype;
    rc = launch(bwd_finalize_kernel_ptr(), dim3((unsigned)cdiv(hidden, 32), ln ? 2 : 1), dim3(256), &fp, st);
    if (rc) return rc;
    return ok();
  }

  if (rows == 0) {
    // nothing to read (the row-indexed pointers may be NULL): the finalize kernel over zero
    // partial rows writes zero gradients
    FinalizeParams fp{};
    fp.part = reinterpret_cast<const float *>(static_cast<char *>(workspace) + kWsHeaderBytes);
    fp.dgamma = dgamma;
    fp.dbeta = ln ? dbeta : nullptr;
    fp.hidden = hidden;
    fp.G = 0;
    fp.w_dtype = w_dtype;
    rc = launch(bwd_finalize_kernel_ptr(), dim3((unsigned)cdiv(hidden, 32), ln ? 2 : 1), dim3(256), &fp, st);
    if (rc) return rc;
    return ok();
  }
  const void *fn = bwd_kernel_ptr(norm_type, in_dtype, with_add, pl.cfg);
  if (!fn) return fail(NORM_ERR_UNSUPPORTED, "no backward kernel for this combination");
  const BwdShape &sh = kBwdShapes[pl.cfg];
  int occ = 1;
  rc = occupancy(fn, sh.threads(), &occ);
  if (rc) return rc;
  const int64_t G = bwd_grid(pl, dev.cus - cu_margin, occ, rows);

  BwdParams p{};
  p.dy = dy;
  p.x = x;
  p.residual = residual;
  p.mu = ln ? mu : nullptr;
  p.rsigma = rsigma;
  p.gamma = gamma;
  p.dx = dx;
  p.part = reinterpret_cast<float *>(static_cast<char *>(workspace) + kWsHeaderBytes);
  p.rows = rows;
  p.hidden = hidden;
  p.w_dtype = w_dtype;
  p.zero_centered = zero_centered_gamma ? 1 : 0;
  p.G = (int)G;
  rc = launch(fn, dim3((unsigned)G), dim3(sh.threads()), &p, st);
  if (rc) return rc;

  FinalizeParams fp{};
  fp.part = p.part;
  fp.dgamma = dgamma;
  fp.dbeta = ln ? dbeta : nullptr;
  fp.hidden = hidden;
  fp.G = (int)G;
  fp.w_dtype = w_dtype;
  rc = launch(bwd_finalize_kernel_ptr(), dim3((unsigned)cdiv(hidden, 32), ln ? 2 : 1), dim3(256), &fp, st);
  if (rc) return rc;
  return ok();
}

int norm_bwd(void *stream, const void *dy, const void *x, const float *mu, const float *rsigma,
             const void *gamma, void *dx, void *dgamma, void *dbeta, void *workspace,
             size_t workspace_bytes, int64_t rows, int64_t hidden, int in_dtype, int w_dtype,
             int norm_type, int zero_centered_gamma, int cu_margin) {
  return bwd_common(stream, false, dy, x, nullptr, mu, rsigma, gamma, dx, dgamma, dbeta, workspace, workspace_bytes,
                    rows, hidden, in_dtype, w_dtype, norm_type, zero_centered_gamma, cu_margin);
}

int norm_bwd_add(void *stream, const void *dy, const void *x, const void *residual_dy, const float *rsigma,
                 const void *gamma, void *dx, void *dgamma, void *workspace, size_t workspace_bytes,
                 int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int zero_centered_gamma,
                 int cu_margin) {
  if (!residual_dy && rows > 0) return fail(NORM_ERR_INVALID_ARG, "residual_dy is required");
  return bwd_common(stream, true, dy, x, residual_dy, nullptr, rsigma, gamma, dx, dgamma, nullptr, workspace,
                    workspace_bytes, rows, hidden, in_dtype, w_dtype, NORM_RMSNORM, zero_centered_gamma,
                    cu_margin);
}

int norm_fwd_launch_shape(int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int out_dtype, int norm_type,
                          int scaling, int qlayout, int cu_margin, int64_t shape[6]) {
  if (!shape) return fail(NORM_ERR_INVALID_ARG, "shape is NULL");
  FwdPlan pl;
  int rc = plan_fwd(rows, hidden, in_dtype, w_dtype, out_dtype, norm_type, scaling, qlayout, cu_margin, &pl);
  if (rc) return rc;
  for (int i = 0; i < 6; ++i) shape[i] = 0;
  shape[5] = 1;
  int route;
  if (pl.gen) route = NORM_ROUTE_GENERAL;
  else if (pl.colx) route = NORM_ROUTE_SINGLE_PASS_COLWISE;
  else if (pl.split) route = NORM_ROUTE_SPLIT;
  else if (pl.band) route = NORM_ROUTE_BAND;
  else if (pl.col) route = pl.tr ? NORM_ROUTE_ROW_TRANSPOSE : NORM_ROUTE_STATS_TILES;
  else route = NORM_ROUTE_ROW;
  shape[0] = route;
  if (route == NORM_ROUTE_ROW || route == NORM_ROUTE_ROW_TRANSPOSE || route == NORM_ROUTE_STATS_TILES) {
    const RowShape &sh = kRowShapes[pl.cfg];
    shape[1] = pl.cfg;
    shape[2] = sh.P;
    shape[3] = sh.KC;
    shape[4] = sh.T;
  } else if (route == NORM_ROUTE_BAND) {
    shape[1] = pl.cfg;
    shape[5] = pl.S;
  } else if (route == NORM_ROUTE_SPLIT) {
    shape[1] = pl.split_shape;
    shape[5] = pl.S;
  } else if (route == NORM_ROUTE_SINGLE_PASS_COLWISE) {
    shape[5] = pl.S;
  }
  return ok();
}

int norm_bwd_launch_shape(int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int norm_type, int with_add,
                          int cu_count, int cu_margin, int occupancy, int64_t shape[5]) {
  if (!shape) return fail(NORM_ERR_INVALID_ARG, "shape is NULL");
  if (with_add && norm_type != NORM_RMSNORM)
    return fail(NORM_ERR_INVALID_ARG, "the fused backward-add is defined for RMSNorm only");
  if (cu_count < 1 || cu_margin < 0 || cu_margin >= cu_count || occupancy < 1)
    return fail(NORM_ERR_INVALID_ARG, "need 0 <= cu_margin < cu_count and occupancy >= 1");
  BwdPlan pl;
  int rc = plan_bwd(rows, hidden, in_dtype, w_dtype, norm_type, cu_margin, &pl);
  if (rc) return rc;
  if (pl.gen) {
    shape[0] = -1;
    shape[1] = shape[2] = shape[3] = shape[4] = 0;
    return ok();
  }
  const BwdShape &sh = kBwdShapes[pl.cfg];
  shape[0] = pl.cfg;
  shape[1] = sh.W;
  shape[2] = sh.KC;
  shape[3] = sh.T;
  shape[4] = bwd_grid(pl, cu_count - cu_margin, occupancy, rows);
  return ok();
}

int norm_tuning_set(const char *name, int value, int *previous) {
  if (!name) return fail(NORM_ERR_INVALID_ARG, "name is NULL");
  knobs_init();
  for (int i = 0; i < K_NKNOBS; ++i) {
    if (strcmp(name, kKnobNames[i]) == 0) {
      const int old = g_knobs[i].exchange(value, std::memory_order_relaxed);
      if (previous) *previous = old;
      return ok();
    }
  }
  return fail(NORM_ERR_INVALID_ARG, "unknown tuning knob %s", name);
}

int norm_workspace_init(void *stream, void *workspace, size_t workspace_bytes) {
  if (!workspace) return fail(NORM_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned16(workspace)) return fail(NORM_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (workspace_bytes < (size_t)kWsHeaderBytes)
    return fail(NORM_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than the %d-byte header", kWsHeaderBytes);
  uint32_t *ws = static_cast<uint32_t *>(workspace);
  void *args[] = {&ws};
  hipError_t e = hipLaunchKernel(ws_init_kernel_ptr(), dim3(1), dim3(256), args, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NORM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int norm_workspace_check(void *stream, void *workspace, uint32_t *flags) {
  if (!workspace || !flags) return fail(NORM_ERR_INVALID_ARG, "workspace and flags are required");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(NORM_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
  static uint32_t words[kWsHeaderBytes / 4];
  static std::mutex mu;
  std::lock_guard<std::mutex> lk(mu);
  e = hipMemcpy(words, workspace, sizeof(words), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(NORM_ERR_HIP, "hipMemcpy: %s", hipGetErrorString(e));
  uint32_t f = words[kWsError];
  // every counter must be back at zero between calls
  bool dirty = words[kWsDone] != 0;
  for (int i = 0; i < kClasses; ++i) dirty |= words[kWsTicket0 + i] != 0;
  for (int i = kWsGroup0; i < kWsAmax0; ++i) dirty |= words[i] != 0;
  if (dirty) f |= 2u;
  *flags = f;
  if (f) {
    e = hipMemset(static_cast<char *>(workspace) + kWsError * 4, 0, 4);
    if (e != hipSuccess) return fail(NORM_ERR_HIP, "hipMemset: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // extern "C"
