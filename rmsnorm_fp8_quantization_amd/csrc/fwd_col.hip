// fwd_col.hip -- second pass of the forward with a columnwise (transposed) FP8 output: given
// each row's statistics, normalise 128 x 128 tiles and write the rowwise and the columnwise
// codes, each as whole 128-byte lines. Also the byte transpose that turns delayed scaling's
// rowwise codes into its columnwise codes (transpose_u8_kernel, at the end of the file).
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization".
// [XLA-Norm] Description: besides the rowwise FP8 output, an optional columnwise output with
// its own scale_inv, for delayed per-tensor scaling and for MXFP8 block scaling. Here the
// columnwise tensor is [hidden, rows] (the transpose), and for MXFP8 each columnwise block is
// 32 consecutive rows of one column.
//
// With CRM (col_rowmajor) the columnwise codes keep the rowwise [rows, hidden] layout (no transpose)
// and the MXFP8 columnwise scales are [ceil(rows/32), hidden].
//
// Two passes: the row kernel first writes mu / rsigma of every row (MODE_STATS); this kernel
// then works on independent tiles. A column of the transposed output is contiguous along
// rows and column pieces shorter than a 128-byte line are not merged on their way to HBM, so
// a tile spans 128 rows; with statistics known in advance no tile waits for another one. The
// price is a second read of x; tiles are visited from the last row down, so the first ones
// read rows the statistics pass streamed most recently (still in the last-level cache).
//
// Work split: a workgroup of 8 waves owns a tile of 128 rows x 128 columns; wave w owns rows
// [16w, 16w + 16); lane l holds rows 16w + 4 (l >> 4) + k (k < 4) of the 8 columns
// 8 (l % 16) + 0..7, so one load instruction covers 4 rows x 256 bytes and one rowwise store
// 4 whole 128-byte lines. The next tile's inputs are loaded while the current tile is
// processed (two register buffers used in turn). FP8 codes of a lane's 4 x 8 block are
// transposed in registers (4 x 4 byte blocks) into its 8 columns' 4-row pieces, staged in LDS
// (two buffers, used in turn) as [column][128 rows] with 16-byte groups XOR-swizzled across
// banks, and stored so that 8 consecutive lanes write a column's 128-byte line. An MXFP8
// columnwise block (32 rows) is two waves: each wave reduces its 16 rows per column and the
// pair combine through LDS. (The tile height kColTileRows is 128; a 256-row
// 16-wave variant whose columns are 256-byte pieces measured slower: one workgroup per
// CU instead of two.)
#include "device_common.hpp"
#include "kernels.hpp"

namespace nf8 {

namespace {

constexpr int kTR = kColTileRows;  // rows per tile (kTR bytes of each column's codes)
constexpr int kTC = kColTileCols;  // 128 columns per tile (one 128-byte line per row)
constexpr int kWaves = kColThreads / 64;  // 16 rows per wave
constexpr int kBlk = kTR / 32;            // MXFP8 columnwise blocks per tile column
constexpr int kLanesPerCol = kTR / 16;    // lanes that store one column's kTR bytes
static_assert((kTR == 128 || kTR == 256) && kTC == 128 && kWaves * 16 == kTR, "tile shape");

// 4 x 4 byte transpose: byte r of word c of the result is byte c of input word r
__device__ __forceinline__ void transpose4x4b(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                              uint32_t (&o)[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// byte offset in a staging buffer of rows [4 piece, 4 piece + 4) of tile column `col`: the
// column's 128 bytes, with its eight 16-byte groups permuted by XOR with (col / 8) % 8
__device__ __forceinline__ int stage_off(int col, int piece) {
  return col * kTR + 4 * (piece ^ (((col >> 3) & 7) << 2));
}

// max over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the same columns in the four row groups)
__device__ __forceinline__ float rowgroup_max(float v) {
  v = fmaxf(v, xor16(v));
  return fmaxf(v, xor32(v));
}

}  // namespace

template <int NORM, class IN, int MODE, bool CRM>
__global__ __launch_bounds__(kColThreads) void fwd_tile_kernel(FwdTileParams tp) {
  static_assert(MODE == MODE_DELAYED || MODE == MODE_MX, "columnwise output is FP8");
  const FwdRowParams &p = tp.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = lane >> 4;  // row group: rows 4 rg .. 4 rg + 3 of the wave
  const int cl = lane & 15;  // columns 8 cl .. 8 cl + 7 of the tile
  const int64_t H = p.hidden;
  const int64_t N = p.rows;
  const int fmt = p.out_dtype;
  const uint32_t tiles_c = (uint32_t)tp.tiles_c;
  const uint32_t ntiles = (uint32_t)(tp.tiles_r * tp.tiles_c);
  // lane offsets within a tile are 32-bit (the planner bounds 128 * hidden * 4 and
  // 128 * rows below 2^32); tile bases are wave-uniform 64-bit pointers
  const uint32_t Hu = (uint32_t)H;
  const uint32_t Nu = (uint32_t)N;
  const int rloc = 16 * wave + 4 * rg;  // this lane's first row within a tile
  const int cloc = 8 * cl;              // this lane's first column within a tile

  __shared__ __align__(16) uint8_t stage[2][kTC * kTR];
  __shared__ __align__(16) float cmax[MODE == MODE_MX ? kWaves : 1][MODE == MODE_MX ? kTC : 4];
  __shared__ uint8_t colx[MODE == MODE_MX ? kBlk : 1][MODE == MODE_MX ? kTC : 1];
  __shared__ uint32_t s_last, s_epoch;
  __shared__ float wred[kColThreads / 64];

  const uint32_t tag = MODE == MODE_DELAYED ? epoch_tag(read_epoch(p.ws, &s_epoch)) : 0u;
  float scale = 1.0f;
  if constexpr (MODE == MODE_DELAYED) scale = *p.scale;
  float amax_local = 0.0f;

  // tile t covers rows [128 rt, +128) and columns [128 ct, +128), visited from the last tile
  struct Tile {
    uint32_t rt, ct;
    int64_t r0, c0;
    int rows_here, cols_here;  // valid rows / columns of the tile (up to 128)
  };
  auto tile_of = [&](uint32_t t) {
    Tile T;
    const uint32_t u = ntiles - 1u - t;
    T.rt = u / tiles_c;
    T.ct = u - T.rt * tiles_c;
    T.r0 = (int64_t)T.rt * kTR;
    T.c0 = (int64_t)T.ct * kTC;
    T.rows_here = (int)(N - T.r0 < kTR ? N - T.r0 : kTR);
    T.cols_here = (int)(H - T.c0 < kTC ? H - T.c0 : kTC);
    return T;
  };

  // This lane's 4 x 8 inputs of tile t. The loads are unconditional (t past the end reads
  // tile 0, rows and columns past the end of a tile read its first row / column) so that no
  // branch makes the number of loads in flight uncertain; what lies outside the tensor is
  // never stored.
  struct TileIn {
    Strip<IN> xs[4];
  };
  auto load_tile = [&](TileIn &d, uint32_t t) {
    const Tile T = tile_of(t < ntiles ? t : 0u);
    const char *xb = static_cast<const char *>(p.x) + (T.r0 * H + T.c0) * IN::bytes;
    const uint32_t co = cloc < T.cols_here ? (uint32_t)cloc : 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t r = rloc + k < T.rows_here ? (uint32_t)(rloc + k) : 0u;
      load_strip<IN>(d.xs[k], xb + (size_t)((r * Hu + co) * (uint32_t)IN::bytes), 0);
    }
  };

  auto step = [&](TileIn &cur, uint32_t t, TileIn &nxt, uint32_t tn, int par) {
    const Tile T = tile_of(t);
    const bool cv = cloc < T.cols_here;
    const int valid = T.rows_here - rloc < 4 ? (T.rows_here - rloc < 0 ? 0 : T.rows_here - rloc) : 4;
    uint8_t *const stg = stage[par];

    // ---- weights and row statistics of this tile, then the next tile's inputs
    float gk[8], bk[8];
    if (cv) {
      load_w8(gk, p.gamma, T.c0 + cloc, p.w_dtype);
      if (p.zero_centered) {
#pragma unroll
        for (int i = 0; i < 8; ++i) gk[i] += 1.0f;
      }
      if constexpr (NORM == NT_LAYERNORM) load_w8(bk, p.beta, T.c0 + cloc, p.w_dtype);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) gk[i] = bk[i] = 0.0f;
    }
    float rs[4], mu[4];
    {
      const float *rsb = tp.st_rs + T.r0;
      const float *mub = tp.st_mu + T.r0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t r = rloc + k < T.rows_here ? (uint32_t)(rloc + k) : 0u;
        rs[k] = rsb[r];
        if constexpr (NORM == NT_LAYERNORM) mu[k] = mub[r];
      }
    }
    load_tile(nxt, tn);

    auto yrow = [&](int k, float (&y)[8]) {
      float xv[8];
      strip_to_f32<IN>(cur.xs[k], xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (NORM == NT_LAYERNORM) y[i] = fmaf((xv[i] - mu[k]) * rs[k], gk[i], bk[i]);
        else y[i] = (xv[i] * rs[k]) * gk[i];
      }
    };

    // ---- MXFP8 columnwise scales: a 32-row block is waves 2b, 2b + 1. For RMSNorm
    // max_r |(x_r rs_r) g| = max_r |x_r rs_r| * |g| exactly (binary32 rounding is monotone), so
    // g is applied once per column.
    float colf[8];
    if constexpr (MODE == MODE_MX) {
      float cm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < valid) {
          if constexpr (NORM == NT_LAYERNORM) {
            float y[8];
            yrow(k, y);
#pragma unroll
            for (int i = 0; i < 8; ++i) cm[i] = fmaxf(cm[i], fabsf(y[i]));
          } else {
            float xv[8];
            strip_to_f32<IN>(cur.xs[k], xv);
#pragma unroll
            for (int i = 0; i < 8; ++i) cm[i] = fmaxf(cm[i], fabsf(xv[i] * rs[k]));
          }
        }
      }
      // converted again below rather than kept live as floats
#pragma unroll
      for (int k = 0; k < 4; ++k) opaque<IN>(cur.xs[k]);
#pragma unroll
      for (int i = 0; i < 8; ++i) cm[i] = rowgroup_max(cm[i]);
      if (rg == 0) {
        float4 *d = reinterpret_cast<float4 *>(&cmax[wave][cloc]);
        d[0] = make_float4(cm[0], cm[1], cm[2], cm[3]);
        d[1] = make_float4(cm[4], cm[5], cm[6], cm[7]);
      }
      __syncthreads();
      const float4 *o = reinterpret_cast<const float4 *>(&cmax[wave ^ 1][cloc]);
      const float4 o0 = o[0], o1 = o[1];
      const float om[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = fmaxf(cm[i], om[i]);
        if constexpr (NORM != NT_LAYERNORM) a = a * fabsf(gk[i]);
        const int X = mx_exponent(a, fmt, p.mx_ceil);
        colf[i] = exp2_neg(X);
        if (rg == 0 && (wave & 1) == 0) colx[wave >> 1][cloc + i] = (uint8_t)(X + 127);
      }
    }

    // ---- codes: rowwise stores; columnwise codes transposed into the staging buffer
    uint8_t *const yb = static_cast<uint8_t *>(p.y) + T.r0 * H + T.c0;
    uint8_t *const sb = MODE == MODE_MX ? static_cast<uint8_t *>(p.scale_inv) + T.r0 * p.mx_cols + (T.c0 >> 5)
                                        : nullptr;
    uint2 codes[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool ok = k < valid && cv;
      uint8_t *const yr = yb + (size_t)((uint32_t)(rloc + k) * Hu + (uint32_t)cloc);
      float y[8];
      yrow(k, y);
      if constexpr (MODE == MODE_DELAYED) {
        float u[8];
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          u[i] = y[i] * scale;
          a = fmaxf(a, fabsf(y[i]));
        }
        if (ok) amax_local = fmaxf(amax_local, a);
        codes[k] = fp8_pack8(u, fmt);
        if (ok && tp.write_row) st_nt8(yr, codes[k]);
      } else {
        if (tp.write_row) {
          float a = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(y[i]));
          a = quad_max(ok ? a : 0.0f);  // 4 lanes = one 32-column block
          const int X = mx_exponent(a, fmt, p.mx_ceil);
          const float f = exp2_neg(X);
          float u[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) u[i] = y[i] * f;
          const uint2 c = fp8_pack8(u, fmt);
          if (ok) {
            st_nt8(yr, c);
            if ((cl & 3) == 0)
              sb[(size_t)((uint32_t)(rloc + k) * (uint32_t)p.mx_cols + (uint32_t)(cloc >> 5))] = (uint8_t)(X + 127);
          }
        }
        float u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = y[i] * colf[i];
        codes[k] = fp8_pack8(u, fmt);
      }
    }
    if constexpr (CRM) {
      // columnwise codes in the rowwise layout: stored like the rowwise codes
      uint8_t *const ycr = static_cast<uint8_t *>(tp.y_col) + T.r0 * H + T.c0;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < valid && cv) st_nt8(ycr + (size_t)((uint32_t)(rloc + k) * Hu + (uint32_t)cloc), codes[k]);
    } else {
      uint32_t lo[4], hi[4];  // lo[i]: column i, hi[i]: column 4 + i; byte k = row k
      transpose4x4b(codes[0].x, codes[1].x, codes[2].x, codes[3].x, lo);
      transpose4x4b(codes[0].y, codes[1].y, codes[2].y, codes[3].y, hi);
      const int piece = 4 * wave + rg;  // rows 4 piece .. 4 piece + 3 of the tile
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint32_t *>(stg + stage_off(cloc + i, piece)) = i < 4 ? lo[i] : hi[i - 4];
    }
    __syncthreads();

    // ---- columnwise stores: thread (c, m) writes rows [16m, 16m + 16) of tile column c
    const bool full = T.rows_here == kTR && (N % 16) == 0;
    uint8_t *const yct = static_cast<uint8_t *>(tp.y_col) + T.c0 * N + T.r0;
    const int m = tid % kLanesPerCol;
#pragma unroll
    for (int pass = 0; pass < (CRM ? 0 : kTC / 64); ++pass) {
      const int c = pass * 64 + tid / kLanesPerCol;
      if (c < T.cols_here) {
        const uint4 v = *reinterpret_cast<const uint4 *>(stg + stage_off(c, 4 * m));
        uint8_t *dst = yct + (size_t)((uint32_t)c * Nu + (uint32_t)(16 * m));
        if (full) {
          st_nt16(dst, v);
        } else {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (16 * m + e < T.rows_here) dst[e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
        }
      }
    }
    if constexpr (MODE == MODE_MX) {
      // the tile's (up to) kBlk 32-row block exponents of each column, consecutive bytes
      if (tid < T.cols_here) {
        const int nb = (T.rows_here + 31) / 32;
        if constexpr (CRM) {  // [ceil(rows/32), hidden] (row stride mx_col_ld): one 128-byte run per block row
          uint8_t *dst = static_cast<uint8_t *>(tp.col_scale_inv) + kBlk * (int64_t)T.rt * tp.mx_col_ld + T.c0 + tid;
          for (int q = 0; q < nb; ++q) dst[(size_t)q * (size_t)tp.mx_col_ld] = colx[q][tid];
        } else {
          uint8_t *dst = static_cast<uint8_t *>(tp.col_scale_inv) + T.c0 * tp.mx_col_ld + kBlk * (int64_t)T.rt +
                         (size_t)((uint32_t)tid * (uint32_t)tp.mx_col_ld);
          if (nb == kBlk && ((uintptr_t)dst & (kBlk - 1)) == 0) {  // one store rather than kBlk byte stores
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int q = 0; q < kBlk; ++q) w[q >> 2] |= (uint32_t)colx[q][tid] << (8 * (q & 3));
            if constexpr (kBlk == 8) *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
            else *reinterpret_cast<uint32_t *>(dst) = w[0];
          } else {
            for (int q = 0; q < nb; ++q) dst[q] = colx[q][tid];
          }
        }
      }
    }
    // No barrier here: the next tile stages into the other buffer, and it rewrites cmax /
    // colx only after its first barrier, which every thread reaches after finishing this tile.
  };

  // two input buffers in turn: tile t is processed while tile t + G loads
  const uint32_t G = gridDim.x;
  TileIn A, B;
  load_tile(A, blockIdx.x);
  for (uint32_t t = blockIdx.x; t < ntiles; t += 2 * G) {
    step(A, t, B, t + G, 0);
    if (t + G >= ntiles) break;
    step(B, t + G, A, t + 2 * G, 1);
  }

  // ---- delayed scaling: tensor amax through the per-workgroup tagged slots
  if constexpr (MODE == MODE_DELAYED) {
    const float m = wave_max(amax_local);
    if (lane == 0) wred[wave] = m;
    __syncthreads();
    if (tid == 0) {
      float a = wred[0];
      for (int w = 1; w < kColThreads / 64; ++w) a = fmaxf(a, wred[w]);
      publish_amax(p.ws, a, tag);
      if (blockIdx.x == 0) {
        if (p.scale_inv) *static_cast<float *>(p.scale_inv) = 1.0f / scale;
        if (tp.col_scale_inv) *static_cast<float *>(tp.col_scale_inv) = 1.0f / scale;
      }
    }
    vmem_drain();
    if (finish_workgroup(p.ws, &s_last)) {
      const float tot = gather_amax(p.ws, gridDim.x, wred, tag);
      if (tid == 0) *p.updated_amax = fmaxf(*p.amax_in, tot);
      vmem_drain();
      __syncthreads();
      reset_completion(p.ws);
    }
  }
}

template <int NORM, class IN>
static const void *pick_tile_mode(int mode, bool crm) {
  switch (mode) {
    case MODE_DELAYED:
      return crm ? (const void *)fwd_tile_kernel<NORM, IN, MODE_DELAYED, true>
                 : (const void *)fwd_tile_kernel<NORM, IN, MODE_DELAYED, false>;
    case MODE_MX:
      return crm ? (const void *)fwd_tile_kernel<NORM, IN, MODE_MX, true>
                 : (const void *)fwd_tile_kernel<NORM, IN, MODE_MX, false>;
    default: return nullptr;
  }
}

template <int NORM>
static const void *pick_tile_in(int in_dtype, int mode, bool crm) {
  switch (in_dtype) {
    case DT_F32: return pick_tile_mode<NORM, F32>(mode, crm);
    case DT_BF16: return pick_tile_mode<NORM, BF16>(mode, crm);
    case DT_F16: return pick_tile_mode<NORM, F16>(mode, crm);
    default: return nullptr;
  }
}

// Columnwise codes of delayed per-tensor scaling as a byte transpose of the rowwise codes the
// row kernel wrote: code(c, r) of the transposed tensor is code(r, c), the same value quantised
// with the same scale. Reads the 256 MiB of rowwise codes instead of the 512 MiB of input a second
// time. A workgroup of 8 waves takes tiles of TR rows x TC columns. A lane holds RL rows of 16
// columns (one 16-byte load per row; TC / 16 lanes cover a tile row, so one load instruction
// covers 64 * 16 / TC rows), transposes them in 4 x 4 byte blocks into its 16 columns' 4-row
// pieces, stages them in LDS as [column][TR rows] (16-byte groups XOR-swizzled as in the tile
// kernel) and stores every column's TR rows as whole lines (TR / 16 lanes x 16 bytes). The next
// tile is loaded while the current one is transposed. Shapes: 512 x 128 (RL = 8, used: 512-byte
// column pieces), 256 x 256 (RL = 8) and 128 x 256 (RL = 4, two staging buffers in turn); one
// staging buffer takes a second barrier. The longer the column pieces, the cheaper the
// transposed writes.
template <int RL, int TC>
__global__ __launch_bounds__(kTrThreads) __attribute__((amdgpu_waves_per_eu(4)))  // two workgroups per CU
void transpose_u8_kernel(TransposeParams tp) {
  static_assert(kTrThreads == 512 && (RL == 4 || RL == 8) && (TC == 256 || (TC == 128 && RL == 8)), "tile shape");
  constexpr int LPR = TC / 16;           // lanes per tile row (16 bytes each)
  constexpr int RG = 64 / LPR;           // row groups per wave
  constexpr int TR = 8 * RG * RL;        // rows per tile: 8 waves x RG groups x RL rows
  constexpr int NBUF = RL == 4 ? 2 : 1;  // staging buffers
  constexpr int LPC = TR / 16;           // lanes per column line
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = lane / LPR;
  const int cl = lane % LPR;
  const int rloc = RG * RL * wave + RL * rg;
  const int cloc = 16 * cl;
  const int64_t H = tp.hidden;
  const int64_t N = tp.rows;
  const uint32_t ntiles = (uint32_t)(tp.tiles_r * tp.tiles_c);
  const uint32_t tiles_c = (uint32_t)tp.tiles_c;
  __shared__ __align__(16) uint8_t stage[NBUF][TC * TR];

  if (blockIdx.x == 0 && tid == 0 && tp.col_scale_inv) *tp.col_scale_inv = 1.0f / *tp.scale;

  struct T2 {
    int64_t r0, c0;
    int rows_here, cols_here;
  };
  auto tile_of = [&](uint32_t t) {
    T2 T;
    const uint32_t rt = t / tiles_c;
    const uint32_t ct = t - rt * tiles_c;
    T.r0 = (int64_t)rt * TR;
    T.c0 = (int64_t)ct * TC;
    T.rows_here = (int)(N - T.r0 < TR ? N - T.r0 : TR);
    T.cols_here = (int)(H - T.c0 < TC ? H - T.c0 : TC);
    return T;
  };
  // loads are unconditional: a tile past the end reads tile 0, rows / columns past the end of a
  // tile read its first row / column (hidden is a multiple of 16, so a 16-byte piece that starts
  // inside the row ends inside it)
  auto load_tile = [&](uint4 (&d)[RL], uint32_t t) {
    const T2 T = tile_of(t < ntiles ? t : 0u);
    const uint8_t *b = tp.src + T.r0 * H + T.c0;
    const int64_t co = cloc < T.cols_here ? cloc : 0;
#pragma unroll
    for (int k = 0; k < RL; ++k) {
      const int64_t r = rloc + k < T.rows_here ? rloc + k : 0;
      d[k] = ld_nt16(b + r * H + co);
    }
  };
  auto soff = [](int col, int piece) {  // 4-row piece `piece` of tile column `col`
    return col * TR + 4 * (piece ^ (((col >> 3) & 7) << 2));
  };
  auto step = [&](uint4 (&cur)[RL], uint32_t t, uint4 (&nxt)[RL], uint32_t tn, int par) {
    const T2 T = tile_of(t);
    load_tile(nxt, tn);
    uint8_t *const stg = stage[NBUF == 2 ? par : 0];
#pragma unroll
    for (int h = 0; h < RL / 4; ++h) {  // rows rloc + 4 h .. + 3: one 4-row piece per column
      const int piece = rloc / 4 + h;
      const uint32_t w0[4] = {cur[4 * h].x, cur[4 * h].y, cur[4 * h].z, cur[4 * h].w};
      const uint32_t w1[4] = {cur[4 * h + 1].x, cur[4 * h + 1].y, cur[4 * h + 1].z, cur[4 * h + 1].w};
      const uint32_t w2[4] = {cur[4 * h + 2].x, cur[4 * h + 2].y, cur[4 * h + 2].z, cur[4 * h + 2].w};
      const uint32_t w3[4] = {cur[4 * h + 3].x, cur[4 * h + 3].y, cur[4 * h + 3].z, cur[4 * h + 3].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // columns cloc + 4 j .. + 3
        uint32_t o[4];
        transpose4x4b(w0[j], w1[j], w2[j], w3[j], o);
#pragma unroll
        for (int c = 0; c < 4; ++c) *reinterpret_cast<uint32_t *>(stg + soff(cloc + 4 * j + c, piece)) = o[c];
      }
    }
    __syncthreads();
    const bool full = T.rows_here == TR && (N % 16) == 0;
    uint8_t *const dt = tp.dst + T.c0 * N + T.r0;
    const int m = tid % LPC;
#pragma unroll
    for (int pass = 0; pass < TC / (kTrThreads / LPC); ++pass) {
      const int c = pass * (kTrThreads / LPC) + tid / LPC;
      if (c < T.cols_here) {
        const uint4 v = *reinterpret_cast<const uint4 *>(stg + soff(c, 4 * m));
        uint8_t *dst = dt + (int64_t)c * N + 16 * m;
        if (full) {
          st_nt16(dst, v);
        } else {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (16 * m + e < T.rows_here) dst[e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
        }
      }
    }
    // two buffers: the next tile stages into the other one; one buffer: wait for every read
    if constexpr (NBUF == 1) __syncthreads();
  };
  const uint32_t G = gridDim.x;
  uint4 A[RL], B[RL];
  load_tile(A, blockIdx.x);
  for (uint32_t t = blockIdx.x; t < ntiles; t += 2 * G) {
    step(A, t, B, t + G, 0);
    if (t + G >= ntiles) break;
    step(B, t + G, A, t + 2 * G, 1);
  }
}

const void *transpose_u8_kernel_ptr(int rows_per_lane, int tile_cols) {
  if (tile_cols == 128) return rows_per_lane == 8 ? (const void *)transpose_u8_kernel<8, 128> : nullptr;
  return rows_per_lane == 8 ? (const void *)transpose_u8_kernel<8, 256> : (const void *)transpose_u8_kernel<4, 256>;
}

const void *fwd_tile_kernel_ptr(int norm, int in_dtype, int mode, bool col_rowmajor) {
  return norm == NT_LAYERNORM ? pick_tile_in<NT_LAYERNORM>(in_dtype, mode, col_rowmajor)
                              : pick_tile_in<NT_RMSNORM>(in_dtype, mode, col_rowmajor);
}

}  // namespace nf8
