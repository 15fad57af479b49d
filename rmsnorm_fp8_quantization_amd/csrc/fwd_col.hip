// fwd_col.hip -- second pass of the forward with a columnwise (transposed) FP8 output: given
// each row's statistics, normalise 128 x 128 tiles and write the rowwise and the columnwise
// codes, each as whole 128-byte lines.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization".
// [XLA-Norm] Description: besides the rowwise FP8 output, an optional columnwise output with
// its own scale_inv, for delayed per-tensor scaling and for MXFP8 block scaling. Here the
// columnwise tensor is [hidden, rows] (the transpose), and for MXFP8 each columnwise block is
// 32 consecutive rows of one column.
//
// Two passes: the row kernel first writes mu / rsigma of every row (MODE_STATS); this kernel
// then works on independent tiles. A column of the transposed output is contiguous along
// rows and column pieces shorter than a 128-byte line are not merged on their way to HBM, so
// a tile spans 128 rows; with statistics known in advance no tile waits for another one,
// which keeps many small workgroups resident per CU. The price is a second read of x.
//
// Work split: a workgroup of 4 waves owns a tile of 128 rows x 128 columns; wave w owns rows
// [32w, 32w + 32); lane l holds rows 32w + 8 (l >> 4) + k (k < 8) of the 8 columns
// 8 (l % 16) + 0..7, so one load instruction covers 4 rows x 256 bytes and one rowwise store
// 4 whole 128-byte lines. FP8 codes of a lane's 8 x 8 block are transposed in registers (4 x 4
// byte blocks) into its 8 columns' 8-row pieces, staged in LDS as [column][128 rows] with the
// pieces XOR-swizzled across banks, and stored so that 8 consecutive lanes write a column's
// 128-byte line. An MXFP8 columnwise block (32 rows) is one wave: its per-column maxima
// combine across the wave's four 16-lane row groups.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nf8 {

namespace {

constexpr int kTR = kColTileRows;  // 128 rows per tile (one 128-byte line per column)
constexpr int kTC = kColTileCols;  // 128 columns per tile (one 128-byte line per row)
static_assert(kTR == 128 && kTC == 128, "tile shape");

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

// byte offset in the staging buffer of rows [8 piece, 8 piece + 8) of tile column `col`
__device__ __forceinline__ int stage_off(int col, int piece) {
  return col * kTR + 8 * (piece ^ ((col >> 3) & 15));
}

// max over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the same columns in the four row groups)
__device__ __forceinline__ float rowgroup_max(float v) {
  v = fmaxf(v, xor16(v));
  return fmaxf(v, xor32(v));
}

// 8 consecutive floats of a per-row array starting at row r (rows >= n read as 0)
__device__ __forceinline__ void load_rows8(float (&o)[8], const float *a, int64_t r, int64_t n) {
  if (r + 8 <= n) {
    const float4 u = *reinterpret_cast<const float4 *>(a + r);
    const float4 v = *reinterpret_cast<const float4 *>(a + r + 4);
    o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w; o[4] = v.x; o[5] = v.y; o[6] = v.z; o[7] = v.w;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = r + k < n ? a[r + k] : 0.0f;
  }
}

}  // namespace

template <int NORM, class IN, int MODE>
__global__ __launch_bounds__(256) void fwd_tile_kernel(FwdTileParams tp) {
  static_assert(MODE == MODE_DELAYED || MODE == MODE_MX, "columnwise output is FP8");
  const FwdRowParams &p = tp.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = lane >> 4;  // row group: rows 8 rg .. 8 rg + 7 of the wave
  const int cl = lane & 15;  // columns 8 cl .. 8 cl + 7 of the tile
  const int64_t H = p.hidden;
  const int64_t N = p.rows;
  const int fmt = p.out_dtype;

  __shared__ __align__(16) uint8_t stage[kTC * kTR];
  __shared__ uint8_t colx[MODE == MODE_MX ? 4 : 1][MODE == MODE_MX ? kTC : 1];
  __shared__ uint32_t s_last, s_epoch;
  __shared__ float wred[4];

  const uint32_t tag = MODE == MODE_DELAYED ? epoch_tag(read_epoch(p.ws, &s_epoch)) : 0u;
  float scale = 1.0f;
  if constexpr (MODE == MODE_DELAYED) scale = *p.scale;
  float amax_local = 0.0f;

  const int64_t ntiles = tp.tiles_r * tp.tiles_c;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t rt = t / tp.tiles_c;
    const int64_t ct = t - rt * tp.tiles_c;
    const int64_t r0 = rt * kTR;                   // first row of the tile
    const int64_t c0 = ct * kTC;                   // first column of the tile
    const int64_t rl = r0 + 32 * wave + 8 * rg;    // first row of this lane
    const int64_t col = c0 + 8 * cl;               // first column of this lane
    const bool cv = col < H;
    const int valid = (int)(N - rl < 8 ? (N - rl < 0 ? 0 : N - rl) : 8);  // this lane's rows

    // ---- inputs
    Strip<IN> xs[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < valid && cv) load_strip<IN>(xs[k], p.x, (rl + k) * H + col);
      else zero_strip<IN>(xs[k]);
    }
    float rs[8], mu[8];
    load_rows8(rs, tp.st_rs, rl, N);
    if constexpr (NORM == NT_LAYERNORM) load_rows8(mu, tp.st_mu, rl, N);
    float gk[8], bk[8];
    if (cv) {
      load_w8(gk, p.gamma, col, p.w_dtype);
      if (p.zero_centered) {
#pragma unroll
        for (int i = 0; i < 8; ++i) gk[i] += 1.0f;
      }
      if constexpr (NORM == NT_LAYERNORM) load_w8(bk, p.beta, col, p.w_dtype);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) gk[i] = bk[i] = 0.0f;
    }
    auto yrow = [&](int k, float (&y)[8]) {
      float xv[8];
      strip_to_f32<IN>(xs[k], xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (NORM == NT_LAYERNORM) y[i] = fmaf((xv[i] - mu[k]) * rs[k], gk[i], bk[i]);
        else y[i] = (xv[i] * rs[k]) * gk[i];
      }
    };

    // ---- MXFP8 columnwise scales: the 32-row block is this wave. For RMSNorm
    // max_r |(x_r rs_r) g| = max_r |x_r rs_r| * |g| exactly (binary32 rounding is monotone), so
    // g is applied once per column.
    float colf[8];
    if constexpr (MODE == MODE_MX) {
      float cm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k < valid) {
          if constexpr (NORM == NT_LAYERNORM) {
            float y[8];
            yrow(k, y);
#pragma unroll
            for (int i = 0; i < 8; ++i) cm[i] = fmaxf(cm[i], fabsf(y[i]));
          } else {
            float xv[8];
            strip_to_f32<IN>(xs[k], xv);
#pragma unroll
            for (int i = 0; i < 8; ++i) cm[i] = fmaxf(cm[i], fabsf(xv[i] * rs[k]));
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = rowgroup_max(cm[i]);
        if constexpr (NORM != NT_LAYERNORM) a = a * fabsf(gk[i]);
        const int X = mx_exponent(a, fmt);
        colf[i] = exp2_neg(X);
        if (rg == 0) colx[wave][8 * cl + i] = (uint8_t)(X + 127);
      }
    }

    // ---- codes: rowwise stores; columnwise codes transposed into the staging buffer
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint2 codes[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k = 4 * h + kk;
        const bool ok = k < valid && cv;
        uint8_t *const yr = static_cast<uint8_t *>(p.y) + (rl + k) * H + col;
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
          codes[kk] = fp8_pack8(u, fmt);
          if (ok && tp.write_row) st_nt8(yr, codes[kk]);
        } else {
          if (tp.write_row) {
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(y[i]));
            a = quad_max(ok ? a : 0.0f);  // 4 lanes = one 32-column block
            const int X = mx_exponent(a, fmt);
            const float f = exp2_neg(X);
            float u[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = y[i] * f;
            const uint2 c = fp8_pack8(u, fmt);
            if (ok) {
              st_nt8(yr, c);
              if ((cl & 3) == 0)
                static_cast<uint8_t *>(p.scale_inv)[(rl + k) * p.mx_cols + (col >> 5)] = (uint8_t)(X + 127);
            }
          }
          float u[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) u[i] = y[i] * colf[i];
          codes[kk] = fp8_pack8(u, fmt);
        }
      }
      uint32_t lo[4], hi[4];  // lo[i]: column i, hi[i]: column 4 + i; byte kk = row 4h + kk
      transpose4x4b(codes[0].x, codes[1].x, codes[2].x, codes[3].x, lo);
      transpose4x4b(codes[0].y, codes[1].y, codes[2].y, codes[3].y, hi);
      const int piece = 4 * wave + rg;  // rows 8 piece .. 8 piece + 7 of the tile
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint32_t *>(stage + stage_off(8 * cl + i, piece) + 4 * h) = i < 4 ? lo[i] : hi[i - 4];
    }
    __syncthreads();

    // ---- columnwise stores: thread (c, m) writes rows [16m, 16m + 16) of tile column c
    {
      const int64_t rows_here = N - r0;  // valid rows of this tile (may be < 128)
      const bool full = rows_here >= kTR && (N % 16) == 0;
      uint8_t *const yct = static_cast<uint8_t *>(tp.y_col) + c0 * N + r0;
      const int m = tid & 7;
#pragma unroll
      for (int pass = 0; pass < kTC / 32; ++pass) {
        const int c = pass * 32 + (tid >> 3);
        if (c0 + c < H) {
          const int slot = (2 * m) ^ ((c >> 3) & 15);  // piece 2m; piece 2m + 1 is at slot ^ 1
          const uint2 a = *reinterpret_cast<const uint2 *>(stage + c * kTR + 8 * slot);
          const uint2 b = *reinterpret_cast<const uint2 *>(stage + c * kTR + 8 * (slot ^ 1));
          uint8_t *dst = yct + (int64_t)c * N + 16 * m;
          if (full) {
            st_nt16(dst, make_uint4(a.x, a.y, b.x, b.y));
          } else {
            const uint32_t w[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (16 * m + e < rows_here) dst[e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
          }
        }
      }
      if constexpr (MODE == MODE_MX) {
        // the tile's (up to) four 32-row block exponents of each column, consecutive bytes
        if (tid < kTC && c0 + tid < H) {
          uint8_t *dst = static_cast<uint8_t *>(tp.col_scale_inv) + (c0 + tid) * tp.mx_rows + 4 * rt;
          const int64_t nb = (rows_here + 31) / 32;
          for (int q = 0; q < 4 && q < nb; ++q) dst[q] = colx[q][tid];
        }
      }
    }
    __syncthreads();  // the staging buffer and colx are rewritten by the next tile
  }

  // ---- delayed scaling: tensor amax through the per-workgroup tagged slots
  if constexpr (MODE == MODE_DELAYED) {
    const float m = wave_max(amax_local);
    if (lane == 0) wred[wave] = m;
    __syncthreads();
    if (tid == 0) {
      publish_amax(p.ws, fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3])), tag);
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
static const void *pick_tile_mode(int mode) {
  switch (mode) {
    case MODE_DELAYED: return (const void *)fwd_tile_kernel<NORM, IN, MODE_DELAYED>;
    case MODE_MX: return (const void *)fwd_tile_kernel<NORM, IN, MODE_MX>;
    default: return nullptr;
  }
}

template <int NORM>
static const void *pick_tile_in(int in_dtype, int mode) {
  switch (in_dtype) {
    case DT_F32: return pick_tile_mode<NORM, F32>(mode);
    case DT_BF16: return pick_tile_mode<NORM, BF16>(mode);
    case DT_F16: return pick_tile_mode<NORM, F16>(mode);
    default: return nullptr;
  }
}

const void *fwd_tile_kernel_ptr(int norm, int in_dtype, int mode) {
  return norm == NT_LAYERNORM ? pick_tile_in<NT_LAYERNORM>(in_dtype, mode) : pick_tile_in<NT_RMSNORM>(in_dtype, mode);
}

}  // namespace nf8
