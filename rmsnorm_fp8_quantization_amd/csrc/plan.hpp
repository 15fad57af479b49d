// plan.hpp -- constants, workspace layout and kernel parameter blocks shared by the host
// launch planner (api.cpp) and the gfx950 kernels.
//
// Pages cited: [XLA-Norm] "Implementation: NVIDIA TransformerEngine JAX XLA Normalization";
// [NVRTC-PR] "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request).
// The pages' dispatch sets grid sizes from device occupancy less an SM margin and keeps
// barrier and workspace buffers for multi-CTA rows ([NVRTC-PR] Flowchart, Greptile Summary;
// [XLA-Norm] Description). This file is the MI355X counterpart: one parameter block per
// kernel family and a fixed workspace header used for cross-workgroup coordination.
#pragma once

#include <stdint.h>

namespace nf8 {

// element-type codes (identical to norm_dtype_t)
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_E4M3 = 3, DT_E5M2 = 4 };
enum : int { NT_LAYERNORM = 0, NT_RMSNORM = 1 };
// epilogue modes (MODE_STATS: statistics only, written to mu / rsigma; no output)
enum : int { MODE_PLAIN = 0, MODE_DELAYED = 1, MODE_MX = 2, MODE_STATS = 3 };

// time limit of a cross-workgroup wait, in ticks of the 100 MHz real-time counter (2 s)
constexpr uint64_t kSpinLimitTicks = 200000000ull;

// ---- workspace header (NORM_WS_HEADER_BYTES at offset 0 of every workspace) --------------
// Counters are zero between calls. A launch that coordinates workgroups counts finished
// workgroups in two levels (64 per group counter, then one counter of finished groups) so no
// word takes more than 64 atomic updates; the workgroup that finishes last publishes the
// per-call results (updated amax), re-zeroes the counters and advances the epoch.
//
// Values that cross workgroups are 64-bit words {value bits, tag} written with one 64-bit
// store; tag = epoch + 1 of the writing launch. A reader polls the words it needs until their
// tag is its own launch's, so it never depends on the order in which two different addresses
// become visible, and a word left by an earlier launch (or a zero-filled workspace) is never
// mistaken for a current one.
constexpr int kWsHeaderBytes = 16384;
constexpr int kWsDone = 0;        // u32: finished groups of workgroups
constexpr int kWsError = 1;       // u32: sticky error flags (bit 0: a wait timed out)
constexpr int kWsEpoch = 2;       // u32: launches completed on this workspace (tags = epoch + 1)
constexpr int kWsTicket0 = 8;     // u32[8]: tile tickets handed out, one counter per class
constexpr int kWsGroup0 = 16;     // u32[32]: finished workgroups per group of 64 (up to word 47)
constexpr int kWsAmax0 = 48;      // u64[kMaxGrid]: per-workgroup {max |y|, tag} (delayed scaling)
constexpr int kWsGroupSize = 64;
constexpr int kMaxGrid = 2016;    // largest persistent grid (bounded by the header's arrays)
constexpr int kClasses = 8;       // ticket classes (one per XCD of the MI355X)
// most workgroups one band may be split over (bounds the LDS used to merge their partials)
constexpr int kMaxSlices = 64;
static_assert(kWsAmax0 * 4 + kMaxGrid * 8 <= kWsHeaderBytes, "header overflow");

// ---- forward row kernel --------------------------------------------------------------------
// A team of P waves normalises one row at a time; a workgroup holds T teams; each lane owns
// KC strips of the row (columns 8 * (team_lane + 64 * P * k), k < KC).
struct FwdRowParams {
  const void *x;
  const void *gamma;
  const void *beta;
  const float *scale;
  const float *amax_in;
  void *y;
  float *mu;
  float *rsigma;
  void *scale_inv;  // delayed: float32[1]; MX: uint8 [rows, ceil(hidden/32)]
  float *updated_amax;
  uint32_t *ws;     // workspace header (delayed scaling) or nullptr
  int64_t rows;
  int64_t hidden;
  int64_t mx_cols;  // row stride of the rowwise E8M0 grid: ceil(hidden / 32), or padded to a multiple of 4
  int w_dtype;
  int out_dtype;    // plain: F32/F16/BF16; delayed / MX: E4M3/E5M2
  int zero_centered;
  int mx_ceil;      // MX: round-up exponent rule (no element saturates) instead of floor
  float eps;
};

// ---- forward band kernel -------------------------------------------------------------------
// A workgroup of 4 waves covers a tile of R = 4 * RW rows x CW = 512 * KC columns; wave w owns
// rows [w * RW, (w + 1) * RW) of the tile and every lane owns KC strips of each of those rows.
// S workgroups cover one band of R full rows and exchange per-row partial statistics through
// the workspace. Used for columnwise outputs and for rows too long for one workgroup.
struct FwdBandParams {
  FwdRowParams f;        // shared fields (y = rowwise output or nullptr)
  void *y_col;           // [hidden, rows] columnwise codes or nullptr
  void *col_scale_inv;   // delayed: float32[1]; MX: uint8 [hidden, ceil(rows/32)]
  uint64_t *partials;    // [bands, S, R, NV] tagged per-row partial statistics (S > 1);
                         // NV = 2 (mean, M2) for LayerNorm, 1 (sum of squares) for RMSNorm
  int64_t bands;         // ceil(rows / R)
  int64_t mx_rows;       // ceil(rows / 32)
  int64_t mx_col_ld;     // row stride of the columnwise E8M0 grid (mx_rows, or padded)
  int S;                 // workgroups per band
  int classes;           // ticket classes (1 or kClasses); gridDim.x is a multiple of it
  int write_row;         // rowwise output requested
};

// ---- forward split kernel (long rows) -------------------------------------------------------
// S workgroups per row group, each holding one slice (16384 or 32768 columns, by shape) of every
// row of the group and that slice's weights (LDS, or gamma in registers); per row the slices
// exchange tagged partial statistics
// (LayerNorm: mean and M2 relative to a shift, and the shift; RMSNorm: the sum of squares).
struct FwdSplitParams {
  FwdRowParams f;        // y = the output
  uint64_t *partials;    // [rows, S, NV] tagged slice partials (NV = 3 LayerNorm, 1 RMSNorm)
  int S;                 // slices per row
};

// ---- forward single-pass columnwise kernel (RMSNorm, FP8) ------------------------------------
// Workgroups own 512-column slices and walk down 128-row bands, exchanging the bands' row sums
// of squares (one tagged word per row and slice) and writing rowwise and columnwise codes.
struct FwdColxParams {
  FwdRowParams f;        // y = rowwise codes (when write_row), scale_inv = rowwise scales
  void *y_col;           // [hidden, rows] columnwise codes
  void *col_scale_inv;   // delayed: float32[1]; MX: uint8 [hidden, rows/32] (row stride mx_col_ld)
  uint64_t *partials;    // [rows / 128, S, 128] tagged slice partials
  int64_t mx_col_ld;
  int S;                 // slices per band (hidden / 512)
  int write_row;
};

// ---- forward tile kernel (second pass of a columnwise output) -------------------------------
// Independent tiles of 128 rows x 128 columns, each normalised with the row statistics the
// first pass (row kernel, MODE_STATS) wrote to st_mu / st_rs.
struct FwdTileParams {
  FwdRowParams f;        // shared fields (y = rowwise output or nullptr)
  void *y_col;           // [hidden, rows] columnwise codes
  void *col_scale_inv;   // delayed: float32[1]; MX: uint8 [hidden, ceil(rows/32)]
  const float *st_mu;    // [rows] (LayerNorm)
  const float *st_rs;    // [rows]
  int64_t mx_rows;       // ceil(rows / 32)
  int64_t mx_col_ld;     // row stride of the columnwise E8M0 grid: mx_rows ([hidden, mx_rows]) or
                         // hidden ([mx_rows, hidden], col_rowmajor), or either padded
  int64_t tiles_r;       // ceil(rows / 128)
  int64_t tiles_c;       // ceil(hidden / 128)
  int write_row;         // rowwise output requested
  int col_rowmajor;      // columnwise output in the [rows, hidden] layout (scales [rows/32, hidden])
};

// ---- byte transpose (columnwise codes of delayed per-tensor scaling) ----------------------
// With one scale for the whole tensor the columnwise codes are the rowwise codes transposed:
// src [rows, hidden] u8 -> dst [hidden, rows] u8, in tiles of 128 (or 256) rows x 256 columns.
struct TransposeParams {
  const uint8_t *src;
  uint8_t *dst;
  const float *scale;    // the tensor scale: colwise_scale_inv = 1 / scale (written once)
  float *col_scale_inv;  // float32[1]
  int64_t rows;
  int64_t hidden;        // a multiple of 16
  int64_t tiles_r;       // ceil(rows / tile rows)
  int64_t tiles_c;       // ceil(hidden / 256)
};

// ---- backward ------------------------------------------------------------------------------
// A workgroup of W waves handles one row at a time (all lanes of the workgroup on one row),
// loops over rows g, g + G, ...; lane owns KC strips (columns 8 * (tid + 64 * W * k)).
// Partial weight gradients of workgroup g, column j go to part[(j / 32) * G + g][j % 32] of a
// [ceil(hidden / 32)][G][32] array (a second one follows for dbeta).
struct BwdParams {
  const void *dy;
  const void *x;
  const void *residual;  // bwd_add or nullptr
  const float *mu;
  const float *rsigma;
  const void *gamma;
  void *dx;
  float *part;           // 1 or 2 arrays [ceil(hidden / 32)][G][32]
  int64_t rows;
  int64_t hidden;
  int w_dtype;
  int zero_centered;
  int G;
};

struct FinalizeParams {
  const float *part;  // 1 or 2 arrays [ceil(hidden / 32)][G][32]
  void *dgamma;
  void *dbeta;        // LayerNorm or nullptr
  int64_t hidden;
  int G;
  int w_dtype;
};

}  // namespace nf8
