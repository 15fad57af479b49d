// fwd_colx.hip -- RMSNorm forward with a columnwise FP8 output (delayed per-tensor or MXFP8
// scaling) in one pass over x: the row statistics of a 128-row band are exchanged between the
// workgroups that hold the band's column slices while the band's data stays in registers.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization";
// [NVRTC-PR] = "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request).
// [XLA-Norm] Description: normalisation and FP8 quantisation in one kernel launch, rowwise with an
// optional columnwise output (delayed tensor scaling or MXFP8 block scaling). [NVRTC-PR] Greptile
// Summary: CTAs that share rows combine their partial statistics through a workspace.
//
// Work split: a workgroup of 8 waves owns a 512-column slice of the tensor and walks down the
// 128-row bands of its group (group = ticket / S, slice = ticket % S, S = hidden / 512). Waves
// 2q, 2q + 1 hold the 128 x 128 sub-tile q of the slice; wave 2q + h holds rows 64h .. 64h + 63;
// lane l holds 16 rows (64h + 16 (l >> 4) + k) of the 8 columns 128q + 8 (l % 16) + i, so one load
// instruction covers 4 rows x 256 bytes and two neighbouring row groups (32 rows) are one MXFP8
// columnwise block. With 8 waves a lane may use 256 registers: two bands of 16 x 8 values and the
// working set fit without spilling. The slice's weights stay in registers for every band.
//
// Per band: every lane's 16 row sums of squares are added over the 16 lanes of its row group and
// over the 4 sub-tiles (LDS, fixed order) into the slice's 128 row partials, published as tagged
// words {value, launch tag}. Every workgroup of the band then sums the S slices' partials of each
// row in one fixed order (four interleaved runs of slices, then the runs), so all S obtain
// identical rsigma. Codes: rowwise from each row's 8 values (an MXFP8 row block is 4 lanes);
// columnwise from each column's 16 values (an MXFP8 column block is 2 row groups of a wave),
// transposed in registers and staged in LDS as [column][128 rows] so that every column of the
// sub-tile is written as one 128-byte line. MXFP8 scales are gathered in LDS and written as one
// 16-byte run per row (16 blocks of the slice) and one 4-byte run per column (the band's 4 blocks).
//
// Two bands are in registers: band j + 1 is reduced and published before band j waits for its
// partners, and band j + 2 loads once band j's codes are out. Every wait has wait_tagged's 2 s limit;
// tickets are taken at start by running workgroups only; the last workgroup re-zeroes the ticket
// counter, gathers the delayed-scaling amax and advances the epoch.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nf8 {

namespace {

constexpr int kXR = 128;   // band height
constexpr int kXQ = 4;     // 128-column sub-tiles per slice

// 4 x 4 byte transpose: byte r of word c of the result is byte c of input word r
__device__ __forceinline__ void xpose4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t (&o)[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// byte offset of rows [4 g, 4 g + 4) of sub-tile column `col` in a [128 columns][128 rows]
// staging buffer: the column's thirty-two 4-byte groups permuted by XOR with a multiple of 4, so
// that a 16-byte piece (groups 4m .. 4m + 3) stays contiguous and in order while the lanes that
// write one row group's columns fall into different banks
__device__ __forceinline__ int xstage(int col, int g) { return col * kXR + 4 * (g ^ (((col >> 3) & 7) << 2)); }

// sum over the 16 lanes of a DPP row (the lanes sharing a row group)
__device__ __forceinline__ float row16_sum(float v) {
  v += xor1(v);
  v += xor2(v);
  v += hmirror(v);
  v += mirror(v);
  return v;
}

}  // namespace

template <class IN, int MODE>
__global__ __launch_bounds__(kColxThreads) void fwd_colx_kernel(FwdColxParams cp) {
  static_assert(MODE == MODE_DELAYED || MODE == MODE_MX, "columnwise output is FP8");
  static_assert(kColxThreads == 512, "8 waves: 2 per 128 x 128 sub-tile");
  constexpr int KR = 16;          // rows per lane
  const FwdRowParams &p = cp.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = wave >> 1;        // sub-tile of the slice
  const int wh = wave & 1;        // 64-row half of the band
  const int rg = lane >> 4;       // row group within the wave
  const int cl = lane & 15;       // column group within the sub-tile
  const int r0 = 64 * wh + KR * rg; // this lane's first row in the band (16 rows)
  const int cs = 128 * q + 8 * cl;  // this lane's first column in the slice (8 columns)
  const int64_t H = p.hidden;
  const int64_t N = p.rows;
  const int S = cp.S;
  const int fmt = p.out_dtype;
  constexpr int TW = kColxCols;
  constexpr int NRUN = kColxThreads / kXR;  // runs of slices in the partial sums

  __shared__ __align__(16) uint8_t stage[kXQ][128 * kXR];
  __shared__ float rpart[2][kXQ][kXR];  // by band parity: a band's partials are read after the
                                        // barrier while the next band's are being written
  __shared__ float rsum[NRUN][kXR];
  __shared__ float rs_l[kXR];
  __shared__ __align__(16) uint8_t rowx[MODE == MODE_MX ? kXR : 1][16];
  __shared__ __align__(4) uint8_t colx[MODE == MODE_MX ? TW : 1][4];
  __shared__ uint32_t s_ticket, s_epoch, s_last;
  __shared__ float wred[kColxThreads / 64];

  if (tid == 0) {
    s_epoch = ld_dev_u32(p.ws + kWsEpoch);
    s_ticket = add_dev(p.ws + kWsTicket0, 1u);
  }
  __syncthreads();
  const uint32_t tag = epoch_tag(s_epoch);
  const int ticket = (int)s_ticket;
  const int group = ticket / S;
  const int slice = ticket - group * S;
  const int ngroups = (int)gridDim.x / S;
  const int64_t c0 = (int64_t)slice * TW;
  const int64_t nbands = N / kXR;
  const int64_t nb = group < nbands ? (nbands - group + ngroups - 1) / ngroups : 0;
  uint32_t *const err = p.ws + kWsError;
  const float inv_h = 1.0f / (float)H;

  float g[8];
  load_w8(g, p.gamma, c0 + cs, p.w_dtype);
  if (p.zero_centered) {
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] += 1.0f;
  }
  float scale = 1.0f;
  if constexpr (MODE == MODE_DELAYED) scale = *p.scale;
  float amax_local = 0.0f;

  auto band_of = [&](int64_t j) { return group + j * ngroups; };
  auto part_of = [&](int64_t b, int s) { return cp.partials + (b * S + s) * (int64_t)kXR; };

  // Addresses are a wave-uniform base (band, slice and row k of the lane's block) plus one 32-bit
  // per-lane offset, so that 16 rows of loads or stores need no 64-bit address per row.
  const uint32_t xoff = (uint32_t)(((int64_t)r0 * H + cs) * IN::bytes);
  const uint32_t yoff = (uint32_t)((int64_t)r0 * H + cs);

  typedef Strip<IN> Tile[KR];
  // band j's 16 x 8 block of this lane (a band past the group's last reads band 0, unused)
  auto load_tile = [&](Tile &t, int64_t j) {
    const int64_t b = j < nb ? band_of(j) : 0;
    const char *base = static_cast<const char *>(p.x) + (b * kXR * H + c0) * IN::bytes;
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const char *rowk = base + (int64_t)k * H * IN::bytes;  // uniform
      load_strip<IN>(t[k], rowk + xoff, 0);
    }
  };

  // ---- band j: the slice's 128 row sums of squares, published
  auto stats_publish = [&](Tile &t, int64_t j) {
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      float xv[8];
      strip_to_f32<IN>(t[k], xv);
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(xv[i], xv[i], s);
      s = row16_sum(s);
      if (cl == 0) rpart[j & 1][q][r0 + k] = s;
    }
#pragma unroll
    for (int k = 0; k < KR; ++k) opaque<IN>(t[k]);
    __syncthreads();
    if (tid < kXR && j < nb) {
      const float(&rp)[kXQ][kXR] = rpart[j & 1];
      const float s = ((rp[0][tid] + rp[1][tid]) + rp[2][tid]) + rp[3][tid];
      st_dev64(part_of(band_of(j), slice) + tid, tagged(s, tag));
    }
  };

  // ---- band j: rsigma from the S slices' partials, then the codes and scales
  auto finish = [&](Tile &t, int64_t j) {
    const int64_t b = band_of(j);
    {
      const int row = tid & (kXR - 1), run = tid / kXR;
      float acc = 0.0f;
      for (int s = run; s < S; s += NRUN) acc += wait_tagged(part_of(b, s) + row, tag, err);
      rsum[run][row] = acc;
    }
    __syncthreads();
    if (tid < kXR) {
      float tot = rsum[0][tid];
#pragma unroll
      for (int r = 1; r < NRUN; ++r) tot += rsum[r][tid];
      const float rsv = __builtin_amdgcn_rsqf(tot * inv_h + p.eps);
      rs_l[tid] = rsv;
      if (slice == 0 && p.rsigma) p.rsigma[b * kXR + tid] = rsv;
    }
    __syncthreads();

    // rowwise codes, row by row; columnwise codes four rows at a time: transposed in registers
    // (4 x 4 bytes) and staged as each column's 4-byte piece of those rows
    uint8_t *const ybase = static_cast<uint8_t *>(p.y) + b * kXR * H + c0;  // uniform
    uint8_t *const stg = stage[q];
    auto stage4 = [&](const uint2 (&c4)[4], int h) {
      uint32_t lo[4], hi[4];  // columns 0..3 and 4..7, rows 4h .. 4h + 3 of the lane's block
      xpose4(c4[0].x, c4[1].x, c4[2].x, c4[3].x, lo);
      xpose4(c4[0].y, c4[1].y, c4[2].y, c4[3].y, hi);
      const int g4 = (r0 >> 2) + h;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        *reinterpret_cast<uint32_t *>(stg + xstage(8 * cl + c, g4)) = lo[c];
        *reinterpret_cast<uint32_t *>(stg + xstage(8 * cl + 4 + c, g4)) = hi[c];
      }
    };
    if constexpr (MODE == MODE_DELAYED) {
      float a = 0.0f;
#pragma unroll
      for (int h = 0; h < KR / 4; ++h) {
        uint2 c4[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int k = 4 * h + kk;
          const float rsk = rs_l[r0 + k];
          float xv[8], u[8];
          strip_to_f32<IN>(t[k], xv);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float y = (xv[i] * rsk) * g[i];
            a = fmaxf(a, fabsf(y));
            u[i] = y * scale;
          }
          c4[kk] = fp8_pack8(u, fmt);  // one scale for the tensor: rowwise and columnwise codes agree
          if (cp.write_row) st_nt8(ybase + (int64_t)k * H + yoff, c4[kk]);
        }
        stage4(c4, h);
      }
      amax_local = fmaxf(amax_local, a);
    } else {
      // rowwise blocks (4 lanes = 32 columns of a row), and each column's maximum over the lane's
      // 16 rows
      float cm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const float rsk = rs_l[r0 + k];
        float xv[8], y[8];
        strip_to_f32<IN>(t[k], xv);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          y[i] = (xv[i] * rsk) * g[i];
          a = fmaxf(a, fabsf(y[i]));
          cm[i] = fmaxf(cm[i], fabsf(y[i]));
        }
        if (cp.write_row) {
          a = quad_max(a);
          const int X = mx_exponent(a, fmt, p.mx_ceil);
          const float f = exp2_neg(X);
          float u[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) u[i] = y[i] * f;
          st_nt8(ybase + (int64_t)k * H + yoff, fp8_pack8(u, fmt));
          if ((cl & 3) == 0) rowx[r0 + k][4 * q + (cl >> 2)] = (uint8_t)(X + 127);
        }
      }
      // columnwise: row groups 2m, 2m + 1 of a wave (32 rows) are one block of a column
      float f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float m = fmaxf(cm[i], xor16(cm[i]));
        const int X = mx_exponent(m, fmt, p.mx_ceil);
        f[i] = exp2_neg(X);
        if ((rg & 1) == 0) colx[cs + i][2 * wh + (rg >> 1)] = (uint8_t)(X + 127);
      }
#pragma unroll
      for (int h = 0; h < KR / 4; ++h) {
        uint2 c4[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int k = 4 * h + kk;
          const float rsk = rs_l[r0 + k];
          float xv[8], u[8];
          strip_to_f32<IN>(t[k], xv);
#pragma unroll
          for (int i = 0; i < 8; ++i) u[i] = ((xv[i] * rsk) * g[i]) * f[i];
          c4[kk] = fp8_pack8(u, fmt);
        }
        stage4(c4, h);
      }
    }
    __syncthreads();
    // every column of the slice: one 128-byte line (8 lanes x 16 bytes) per sub-tile column (a
    // uniform base per sub-tile and half, plus the lane's 32-bit offset)
    {
      const int m = tid & 7;
      const uint32_t loff = (uint32_t)(tid >> 3) * (uint32_t)N + 16u * (uint32_t)m;
      uint8_t *const cbase = static_cast<uint8_t *>(cp.y_col) + c0 * N + b * kXR;
#pragma unroll
      for (int qq = 0; qq < kXQ; ++qq) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int col = (tid >> 3) + 64 * hh;
          const uint4 v = *reinterpret_cast<const uint4 *>(stage[qq] + xstage(col, 4 * m));
          st_nt16(cbase + (int64_t)(128 * qq + 64 * hh) * N + loff, v);
        }
      }
    }
    if constexpr (MODE == MODE_MX) {
      {  // the band's 4 block exponents of column tid: one 4-byte run
        uint8_t *dst = static_cast<uint8_t *>(cp.col_scale_inv) + c0 * cp.mx_col_ld + 4 * b +
                       (uint32_t)tid * (uint32_t)cp.mx_col_ld;
        *reinterpret_cast<uint32_t *>(dst) = *reinterpret_cast<const uint32_t *>(colx[tid]);
      }
      if (cp.write_row && tid < kXR) {  // the slice's 16 block exponents of row tid: one 16-byte run
        uint8_t *dst = static_cast<uint8_t *>(p.scale_inv) + (b * kXR + tid) * p.mx_cols + c0 / 32;
        *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(rowx[tid]);
      }
    }
  };

  // two bands in registers: band j + 1 is reduced and published before band j waits for its
  // partners, band j + 2 loads once band j's codes are out
  Tile A, B;
  load_tile(A, 0);
  load_tile(B, 1);
  stats_publish(A, 0);
  for (int64_t j = 0; j < nb; j += 2) {
    stats_publish(B, j + 1);
    finish(A, j);
    load_tile(A, j + 2);
    if (j + 1 >= nb) break;
    stats_publish(A, j + 2);
    finish(B, j + 1);
    load_tile(B, j + 3);
  }

  // ---- end of launch
  if constexpr (MODE == MODE_DELAYED) {
    const float m = wave_max(amax_local);
    if (lane == 0) wred[wave] = m;
    __syncthreads();
    if (tid == 0) {
      float a = wred[0];
      for (int w = 1; w < kColxThreads / 64; ++w) a = fmaxf(a, wred[w]);
      publish_amax(p.ws, a, tag);
      if (blockIdx.x == 0) {
        if (p.scale_inv) *static_cast<float *>(p.scale_inv) = 1.0f / scale;
        if (cp.col_scale_inv) *static_cast<float *>(cp.col_scale_inv) = 1.0f / scale;
      }
    }
  }
  vmem_drain();
  if (finish_workgroup(p.ws, &s_last)) {
    if constexpr (MODE == MODE_DELAYED) {
      const float tot = gather_amax(p.ws, gridDim.x, wred, tag);
      if (tid == 0) *p.updated_amax = fmaxf(*p.amax_in, tot);
    }
    if (tid == 0) xchg_dev(p.ws + kWsTicket0, 0u);
    vmem_drain();
    __syncthreads();
    reset_completion(p.ws);
  }
}

template <class IN>
static const void *pick_colx_mode(int mode) {
  switch (mode) {
    case MODE_DELAYED: return (const void *)fwd_colx_kernel<IN, MODE_DELAYED>;
    case MODE_MX: return (const void *)fwd_colx_kernel<IN, MODE_MX>;
    default: return nullptr;
  }
}

const void *fwd_colx_kernel_ptr(int in_dtype, int mode) {
  switch (in_dtype) {
    case DT_F32: return pick_colx_mode<F32>(mode);
    case DT_BF16: return pick_colx_mode<BF16>(mode);
    case DT_F16: return pick_colx_mode<F16>(mode);
    default: return nullptr;
  }
}

}  // namespace nf8
