// kernels.hpp -- kernel variants compiled into the library and the lookup functions the host
// planner uses to obtain them (as `const void*` for hipLaunchKernel / occupancy queries).
#pragma once

#include "plan.hpp"

namespace nf8 {

// ---- forward row kernel: team of P waves per row, T teams per workgroup, KC strips per lane
enum RowCfg : int {
  ROW_W1_K1 = 0,
  ROW_W1_K2,
  ROW_W1_K4,
  ROW_W1_K8,
  ROW_W4_K2,
  ROW_W4_K4,
  ROW_W8_K4,
  ROW_W2T2_K4,  // 2 waves per row, 2 rows per workgroup
  ROW_W8_K1,
  ROW_W4T2_K2,  // 4 waves per row, 2 rows per workgroup
  ROW_W16_K8,   // 16 waves per row (long rows, weights read from the caches per strip)
  ROW_W4T4_K4,  // 4 waves per row, 4 rows per workgroup: the rows share the LDS weights
  ROW_W16_K2,   // 16 waves per row, 2 strips per lane (RMSNorm rows of 8193..16384)
  ROW_W8T2_K4,  // 8 waves per row, 2 rows per workgroup sharing 128 KB of LDS weights
  ROW_W16_K4,   // 16 waves per row, 4 strips per lane (rows of 16385..32768)
  ROW_W8_K8,    // 8 waves per row, 8 strips per lane, gamma and beta in registers (LayerNorm rows of
                // 16385..32768, 16-bit input, no FP8 epilogue; instantiated for 16-bit plain and
                // statistics-only passes only)
  ROW_W4_K8,    // 4 waves per row, 8 strips per lane, gamma and beta in registers (LayerNorm rows of
                // 8193..16384, the same instances)
  ROW_NCFG
};
struct RowShape {
  int P, T, KC;
  int threads() const { return 64 * P * T; }
  int64_t cover() const { return 512LL * P * KC; }  // row elements one team holds
};
constexpr RowShape kRowShapes[ROW_NCFG] = {{1, 4, 1}, {1, 4, 2}, {1, 4, 4}, {1, 4, 8}, {4, 1, 2}, {4, 1, 4},
                                           {8, 1, 4}, {2, 2, 4}, {8, 1, 1}, {4, 2, 2}, {16, 1, 8},
                                           {4, 4, 4}, {16, 1, 2}, {8, 2, 4}, {16, 1, 4}, {8, 1, 8}, {4, 1, 8}};

// ---- forward band kernel: 4 waves, RW rows per wave, KC strips per lane
enum BandCfg : int { BAND_R8_K1 = 0, BAND_R8_K2, BAND_R4_K2, BAND_R1_K4, BAND_R2_K8, BAND_NCFG };
struct BandShape {
  int RW, KC;
  bool colwise_ok;
  int rows() const { return 4 * RW; }
  int64_t cols() const { return 512LL * KC; }
};
constexpr BandShape kBandShapes[BAND_NCFG] = {{8, 1, true}, {8, 2, true}, {4, 2, true}, {1, 4, false}, {2, 8, false}};

// ---- backward: W waves per row, KC strips per lane
enum BwdCfg : int {
  BWD_W2_K1 = 0,
  BWD_W4_K1,
  BWD_W4_K2,
  BWD_W8_K2,
  BWD_W16_K2,
  BWD_W8_K1,
  BWD_W16_K1,
  BWD_W4_K4,
  BWD_W2_K1_T1,  // one-team twins of the first three, for few rows per workgroup
  BWD_W4_K1_T1,
  BWD_W4_K2_T1,
  BWD_W8_K3,     // 8 waves x 3 strips: rows up to 12288 with the next row in flight
  BWD_W5_K2_T2,  // 5 waves x 2 strips, two teams: an exact cover of 5120-element rows
  BWD_W5_K2_T1,  // its one-team twin
  BWD_NCFG
};
// T teams of W waves per workgroup, each team on its own row; the teams share one partial
// row of weight gradients, so the workgroup count (and the partial traffic) stays one per CU
struct BwdShape {
  int W, KC, T;
  constexpr int threads() const { return 64 * W * T; }
  constexpr int64_t cover() const { return 512LL * W * KC; }
};
// (shape constants are fixed here, not overridable per translation unit: the planner in api.cpp
// and the kernels must agree on every team count, thread count and tile size)
constexpr BwdShape kBwdShapes[BWD_NCFG] = {{2, 1, 4}, {4, 1, 2}, {4, 2, 2}, {8, 2, 1},
                                           {16, 2, 1}, {8, 1, 1}, {16, 1, 1}, {4, 4, 1},
                                           {2, 1, 1}, {4, 1, 1}, {4, 2, 1}, {8, 3, 1},
                                           {5, 2, 2}, {5, 2, 1}};

// ---- forward split kernel: S workgroups per row, each holding one slice of every row of its row
// group. Shape 0 (any input dtype): 16 waves x 2 strips, a 16384-column slice, its weights in
// LDS, four rows in flight. Shape 1 (16-bit input): 8 waves x 8 strips, a 32768-column slice,
// gamma in registers and beta (LayerNorm) in LDS, three rows in flight. Shape 2 (16-bit input):
// 8 waves x 4 strips, a 16384-column slice, gamma in registers and beta in LDS, four rows in
// flight.
struct SplitShape {
  int threads, strips, wreg, depth;
  constexpr int64_t cols() const { return 8LL * threads * strips; }
};
constexpr SplitShape kSplitShapes[3] = {{1024, 2, 0, 4}, {512, 8, 1, 3}, {512, 4, 1, 4}};
constexpr int kSplitMaxSlices = 8;  // shapes 0 and 2: rows up to 131072 elements; shape 1: 262144

// ---- single-pass columnwise kernel: 8 waves, 128-row bands of 512-column slices
constexpr int kColxThreads = 512;
constexpr int kColxCols = 512;
constexpr int kColxRows = 128;

// ---- forward tile kernel (second pass of a columnwise output): 8 waves, 128 x 128 tiles
constexpr int kColTileRows = 128;
constexpr int kColTileCols = 128;
constexpr int kColThreads = 4 * kColTileRows;  // 16 rows per wave

const void *fwd_row_kernel_ptr(int norm, int in_dtype, int mode, int cfg);
const void *fwd_band_kernel_ptr(int norm, int in_dtype, int mode, bool col, int cfg);
const void *fwd_split_kernel_ptr(int norm, int in_dtype, int shape);  // shape 1: 16-bit input only
const void *fwd_colx_kernel_ptr(int in_dtype, int out_dtype, int mode);  // RMSNorm only
const void *fwd_tile_kernel_ptr(int norm, int in_dtype, int mode, bool col_rowmajor);
// tiles of 32 * rows_per_lane rows x 256 columns (rows_per_lane 4 or 8), or of 512 rows x 128
// columns (tile_cols 128, rows_per_lane 8)
const void *transpose_u8_kernel_ptr(int rows_per_lane, int tile_cols);
constexpr int kTrThreads = 512;
// general kernels (any hidden size, element-aligned tensors)
const void *fwd_gen_row_kernel_ptr(int norm, int in_dtype, int mode);
const void *fwd_gen_col_kernel_ptr(int norm, int in_dtype, int mode, bool col_rowmajor);
const void *bwd_gen_row_kernel_ptr(int norm, int in_dtype, bool add);
const void *bwd_gen_wgrad_kernel_ptr(int norm, int in_dtype);
const void *bwd_kernel_ptr(int norm, int in_dtype, bool add, int cfg);
const void *bwd_finalize_kernel_ptr();
const void *ws_init_kernel_ptr();

// host side: record `msg` as the calling thread's norm_last_error() and return `code`
int set_last_error(int code, const char *msg);

}  // namespace nf8
