// fwd_colx.hip -- RMSNorm forward with a columnwise FP8 output (delayed per-tensor or MXFP8
// scaling) in one pass over x: the row statistics of a band are exchanged between the
// workgroups that hold the band's column slices while the band's data stays on chip.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization";
// [NVRTC-PR] = "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request).
// [XLA-Norm] Description: normalisation and FP8 quantisation in one kernel launch, rowwise with an
// optional columnwise output (delayed tensor scaling or MXFP8 block scaling). [NVRTC-PR] Greptile
// Summary: CTAs that share rows combine their partial statistics through a workspace.
//
// Work split: a workgroup of 8 waves owns a 512-column slice of the tensor and walks down the
// 128-row super-bands of its group (group = ticket / S, slice = ticket % S, S = hidden / 512),
// each as two 64-row bands, one per step. Waves 2q, 2q + 1 hold the 64 x 128 sub-tile q of the
// slice; wave 2q + h holds rows 32h .. 32h + 31; lane l holds 8 rows (32h + 8 (l >> 4) + k) of the 8
// columns 128q + 8 (l % 16) + i, so one load instruction covers 4 rows x 256 bytes and a wave's 32
// rows are one MXFP8 columnwise block.
//
// Pipeline: four bands are in registers (32 registers each for 16-bit input). At step j the codes
// of band j are computed, the row sums of band j + 2 are published, and band j + 3 is loaded: a
// band's loads have two steps to land and its partials two steps to reach the other slices.
// One wave's memory counter retires in issue order, so a poll of the partner slices' words would
// also wait for every load and store the wave has in flight. Waves 0-1 therefore poll (two
// threads per row, each over half of the slices) and issue their loads only afterwards; waves 2-7
// issue theirs before the poll; waves 2-3 publish; waves 4-7 write every output from LDS, so the
// polling waves never wait on a store.
//
// Per band: every lane's 8 row sums of squares are added over the 16 lanes of its row group and
// over the 4 sub-tiles (LDS, fixed order) into the slice's 64 row partials, published as tagged
// words {value, launch tag}. Every workgroup of the band adds each row's S partials in the same
// fixed order, so all S obtain identical rsigma. Codes: rowwise from each row's 8 values (an
// MXFP8 row block is 4 lanes), columnwise from each column's 8 values (an MXFP8 column block is a
// wave's 4 row groups), transposed in registers. Both are staged in LDS: rows are written per band
// as 512-byte runs; columns once per super-band, as one 128-byte line per column; MXFP8 scales as
// one 16-byte run per row (the slice's 16 blocks) and one 4-byte run per column (the super-band's
// 4 blocks). Every wait has wait_tagged's 2 s limit; tickets are taken at start by running
// workgroups only; the last workgroup re-zeroes the ticket counter, gathers the delayed-scaling
// amax and advances the epoch.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nf8 {

namespace {

constexpr int kXB = 64;    // band height (one step)
constexpr int kXS = 128;   // super-band height (one columnwise line)
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

// byte offset of super-band rows [4 g, 4 g + 4) of sub-tile column `col` in a
// [128 columns][128 rows] staging buffer: the column's thirty-two 4-byte groups permuted by XOR
// with a multiple of 4, so that a 16-byte piece (groups 4m .. 4m + 3) stays contiguous and in order
// while the lanes that write one row group's columns fall into different banks
__device__ __forceinline__ int xstage(int col, int g) { return col * kXS + 4 * (g ^ (((col >> 3) & 7) << 2)); }

// row-code staging [64 rows][512 bytes]: 128-byte halves swapped between neighbouring row
// groups (bank spread); a 16-byte piece stays whole
__device__ __forceinline__ int rsw(int r) { return ((r >> 3) & 1) << 7; }

// sum over the 16 lanes of a DPP row (the lanes sharing a row group)
__device__ __forceinline__ float row16_sum(float v) {
  v += xor1(v);
  v += xor2(v);
  v += hmirror(v);
  v += mirror(v);
  return v;
}

// a new definition of a strip's registers without an instruction: the value a tile held before
// is dead from here on, though the compiler cannot see that every path reloads the tile
template <class T> __device__ __forceinline__ void fresh(Strip<T> &s) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(Strip<T>) / 16); ++i)
    asm volatile("" : "=v"(s.v[i].x), "=v"(s.v[i].y), "=v"(s.v[i].z), "=v"(s.v[i].w));
}

}  // namespace

template <class IN, int MODE, int FMT>
__global__ __launch_bounds__(kColxThreads) void fwd_colx_kernel(FwdColxParams cp) {
  static_assert(MODE == MODE_DELAYED || MODE == MODE_MX, "columnwise output is FP8");
  static_assert(kColxThreads == 512 && kColxRows == kXS && kColxCols == 512, "8 waves: 2 per 64 x 128 sub-tile");
  constexpr int KR = 8;           // rows per lane
  const FwdRowParams &p = cp.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: role tests branch on it)
  const int q = wave >> 1;        // sub-tile of the slice
  const int wh = wave & 1;        // 32-row half of the band
  const int rg = lane >> 4;       // row group within the wave
  const int cl = lane & 15;       // column group within the sub-tile
  const int r0 = 32 * wh + KR * rg; // this lane's first row in the band (8 rows)
  const int cs = 128 * q + 8 * cl;  // this lane's first column in the slice (8 columns)
  const int64_t H = p.hidden;
  const int64_t N = p.rows;
  const int S = cp.S;
  constexpr int fmt = FMT;  // (a compile-time format: one conversion path, no selects)
  constexpr int TW = kColxCols;
  constexpr int kPollWaves = 2, kPubWave0 = 2, kStoreWave0 = 4;
  constexpr int ST = kColxThreads - 64 * kStoreWave0;  // storing threads (256)

  __shared__ __align__(16) uint8_t stage[kXQ][128 * kXS];  // column codes, [column][128 rows] per sub-tile
  __shared__ __align__(16) uint8_t rstage[kXB][TW];        // row codes, [row][512 columns]
  __shared__ float rpart[kXQ][kXB];
  __shared__ float psum[2][2][kXB];                        // [band parity][half of the slices][row]
  __shared__ __align__(16) uint8_t rowx[MODE == MODE_MX ? kXB : 1][16];
  __shared__ __align__(4) uint8_t colx[MODE == MODE_MX ? TW : 1][4];
  __shared__ uint32_t s_ticket, s_epoch, s_last;
  __shared__ float wred[kColxThreads / 64];
  __shared__ __align__(16) float wl[TW];

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
  const int64_t nsb = N / kXS;
  const int64_t nb = group < nsb ? 2 * ((nsb - group + ngroups - 1) / ngroups) : 0;  // bands (steps)
  uint32_t *const err = p.ws + kWsError;
  const float inv_h = 1.0f / (float)H;
  const int Sh = (S + 1) >> 1;  // slices added by the first poll thread of a row

  // the slice's weights (g = gamma, or 1 + gamma) in LDS: each pass over a band reads its 8
  {
    float g0[8];
    load_w8(g0, p.gamma, c0 + cs, p.w_dtype);
    if (p.zero_centered) {
#pragma unroll
      for (int i = 0; i < 8; ++i) g0[i] += 1.0f;
    }
    if (wh == 0 && rg == 0) {
      *reinterpret_cast<float4 *>(&wl[cs]) = make_float4(g0[0], g0[1], g0[2], g0[3]);
      *reinterpret_cast<float4 *>(&wl[cs + 4]) = make_float4(g0[4], g0[5], g0[6], g0[7]);
    }
  }
  auto load_g = [&](float (&g)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(&wl[cs]);
    const float4 c = *reinterpret_cast<const float4 *>(&wl[cs + 4]);
    g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w; g[4] = c.x; g[5] = c.y; g[6] = c.z; g[7] = c.w;
  };
  float scale = 1.0f;
  if constexpr (MODE == MODE_DELAYED) scale = *p.scale;
  float amax_local = 0.0f;

  // step j: 64-row band 2 sb + (j & 1) of super-band sb = group + (j >> 1) ngroups
  auto band_of = [&](int64_t j) { return 2 * (group + (j >> 1) * ngroups) + (j & 1); };
  auto part_of = [&](int64_t bj, int s) { return cp.partials + (bj * S + s) * (int64_t)kXB; };
  // rsigma of row r of band j from the two poll threads' sums (one fixed order everywhere)
  auto rs_of = [&](int64_t j, int r) {
    return __builtin_amdgcn_rsqf((psum[j & 1][0][r] + psum[j & 1][1][r]) * inv_h + p.eps);
  };

  // Addresses are a wave-uniform base plus one 32-bit per-lane offset, so that the rows of a load
  // need no 64-bit address per row.
  const uint32_t xoff = (uint32_t)(((int64_t)r0 * H + cs) * IN::bytes);

  typedef Strip<IN> Tile[KR];
  auto load_tile = [&](Tile &t, int64_t j) {
    const char *base = static_cast<const char *>(p.x) + (band_of(j) * kXB * H + c0) * IN::bytes;
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const char *rowk = base + (int64_t)k * H * IN::bytes;  // uniform
      load_strip<IN>(t[k], rowk + xoff, 0);
    }
  };

  // ---- the slice's 64 row sums of squares of a loaded band, into rpart (read after a barrier)
  auto row_sums = [&](Tile &t) {
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      float s = strip_sumsq<IN>(t[k]);
      s = row16_sum(s);
      if (cl == 0) rpart[q][r0 + k] = s;
    }
#pragma unroll
    for (int k = 0; k < KR; ++k) opaque<IN>(t[k]);
  };
  // waves 2-3: band j's partials, published
  auto publish = [&](int64_t j) {
    const int row = tid - 64 * kPubWave0;
    if (row >= 0 && row < kXB) {
      const float s = ((rpart[0][row] + rpart[1][row]) + rpart[2][row]) + rpart[3][row];
      st_dev64(part_of(band_of(j), slice) + row, tagged(s, tag));
    }
  };
  // waves 0-1: thread (h, row) adds row's partials of slices [h Sh, min(S, (h + 1) Sh)) of band j in
  // slice order (loads issued 16 at a time before any tag is looked at; only a word not yet tagged
  // with this launch is polled again)
  auto poll = [&](int64_t j) {
    const int row = tid & (kXB - 1), h = tid >> 6;
    const char *const pb = reinterpret_cast<const char *>(part_of(band_of(j), 0));  // uniform
    auto word = [&](int s_) { return reinterpret_cast<const uint64_t *>(pb + (uint32_t)(s_ * kXB + row) * 8u); };
    const int s_lo = h * Sh, s_hi = S < s_lo + Sh ? S : s_lo + Sh;
    constexpr int PB = 16;
    float acc = 0.0f;
    for (int s0 = s_lo; s0 < s_hi; s0 += PB) {
      uint64_t v[PB];
#pragma unroll
      for (int i = 0; i < PB; ++i) v[i] = ld_dev64(word(s0 + i < s_hi ? s0 + i : s_lo));
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        if (s0 + i < s_hi) {
          const float x = (uint32_t)(v[i] >> 32) == tag ? __uint_as_float((uint32_t)v[i])
                                                         : wait_tagged(word(s0 + i), tag, err);
          acc += x;
        }
      }
    }
    psum[j & 1][h][row] = acc;
  };

  // ---- band j's codes (and MXFP8 scales) into LDS
  auto codes = [&](Tile &t, int64_t j) {
    float g[8];
    load_g(g);
    float rs[KR];
#pragma unroll
    for (int k = 0; k < KR; ++k) rs[k] = rs_of(j, r0 + k);
    uint8_t *const stg = stage[q];
    const int gbase = (kXB * (int)(j & 1) + r0) >> 2;  // the lane's first 4-row group in the super-band
    // columnwise codes four rows at a time: transposed in registers (4 x 4 bytes) and staged as
    // each column's 4-byte piece of those rows
    auto stage4 = [&](const uint2 (&c4)[4], int h) {
      uint32_t lo[4], hi[4];  // columns 0..3 and 4..7, rows 4h .. 4h + 3 of the lane's block
      xpose4(c4[0].x, c4[1].x, c4[2].x, c4[3].x, lo);
      xpose4(c4[0].y, c4[1].y, c4[2].y, c4[3].y, hi);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        *reinterpret_cast<uint32_t *>(stg + xstage(8 * cl + c, gbase + h)) = lo[c];
        *reinterpret_cast<uint32_t *>(stg + xstage(8 * cl + 4 + c, gbase + h)) = hi[c];
      }
    };
    // (the lane's 8 rows share one swizzle: r0 is a multiple of 8)
    uint8_t *const rsl = &rstage[0][0] + r0 * TW + (cs ^ rsw(r0));
    auto stage_row = [&](int k, uint2 v) { *reinterpret_cast<uint2 *>(rsl + k * TW) = v; };
    if constexpr (MODE == MODE_DELAYED) {
      float a = 0.0f;
#pragma unroll
      for (int h = 0; h < KR / 4; ++h) {
        uint2 c4[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int k = 4 * h + kk;
          float xv[8], u[8];
          strip_to_f32<IN>(t[k], xv);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float y = (xv[i] * rs[k]) * g[i];
            a = fmaxf(a, fabsf(y));
            u[i] = y * scale;
          }
          c4[kk] = fp8_pack8(u, fmt);  // one scale for the tensor: rowwise and columnwise codes agree
          if (cp.write_row) stage_row(k, c4[kk]);
        }
        stage4(c4, h);
      }
      amax_local = fmaxf(amax_local, a);
    } else {
      // pass 1: each row block's exponent (4 lanes = 32 columns of a row) into rowx, and each
      // column's maximum over the lane's 8 rows
      float cm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        float xv[8];
        strip_to_f32<IN>(t[k], xv);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float y = (xv[i] * rs[k]) * g[i];
          a = fmaxf(a, fabsf(y));
          cm[i] = fmaxf(cm[i], fabsf(y));
        }
        if (cp.write_row) {
          a = quad_max(a);
          const int X = mx_exponent(a, fmt, p.mx_ceil);
          if ((cl & 3) == 0) rowx[r0 + k][4 * q + (cl >> 2)] = (uint8_t)(X + 127);
        }
      }
      // columnwise: a wave's 4 row groups (32 rows) are one block of a column, block
      // 2 (j & 1) + wh of the super-band
      float f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float m = fmaxf(cm[i], xor16(cm[i]));
        m = fmaxf(m, xor32(m));
        const int X = mx_exponent(m, fmt, p.mx_ceil);
        f[i] = exp2_neg(X);
        if (rg == 0) colx[cs + i][2 * (int)(j & 1) + wh] = (uint8_t)(X + 127);
      }
      // pass 2: both codes of each value (the row block's exponent read back from rowx, written
      // above by a lane of the same wave: the read names the written address, so it stays after
      // the write, and a wave's LDS accesses complete in order)
#pragma unroll
      for (int h = 0; h < KR / 4; ++h) {
        uint2 c4[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int k = 4 * h + kk;
          float xv[8], y[8], u[8];
          strip_to_f32<IN>(t[k], xv);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            y[i] = (xv[i] * rs[k]) * g[i];
            u[i] = y[i] * f[i];
          }
          c4[kk] = fp8_pack8(u, fmt);
          if (cp.write_row) {
            const float fr = exp2_neg((int)rowx[r0 + k][4 * q + (cl >> 2)] - 127);
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = y[i] * fr;
            stage_row(k, fp8_pack8(u, fmt));
          }
        }
        stage4(c4, h);
      }
    }
  };

  // ---- waves 4-7: band j's outputs from LDS; the columnwise lines and scales of the super-band
  // after its second band (a uniform base per step plus a 32-bit lane offset)
  auto store = [&](int64_t j) {
    const int t = tid - 64 * kStoreWave0;
    const int64_t bj = band_of(j);
    if (cp.write_row) {  // 8 rows x 512 bytes per step
      uint8_t *const ybase = static_cast<uint8_t *>(p.y) + bj * kXB * H + c0;
      const uint32_t loff = (uint32_t)(t >> 5) * (uint32_t)H + 16u * (uint32_t)(t & 31);
#pragma unroll 4
      for (int it = 0; it < kXB * TW / 16 / ST; ++it) {
        const int r = it * (ST / 32) + (t >> 5);
        const uint4 v = *reinterpret_cast<const uint4 *>(&rstage[r][(16 * (t & 31)) ^ rsw(r)]);
        st_nt16(ybase + (int64_t)it * (ST / 32) * H + loff, v);
      }
      if constexpr (MODE == MODE_MX) {
        if (t < kXB) {  // the slice's 16 block exponents of row t: one 16-byte run
          uint8_t *dst = static_cast<uint8_t *>(p.scale_inv) + (bj * kXB + t) * p.mx_cols + c0 / 32;
          *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(rowx[t]);
        }
      }
    }
    if (slice == 0 && p.rsigma && t >= kXB && t < 2 * kXB) p.rsigma[bj * kXB + t - kXB] = rs_of(j, t - kXB);
    if (j & 1) {
      const int64_t sb = bj >> 1;
      {  // 32 columns x 128 bytes per step
        uint8_t *const cbase = static_cast<uint8_t *>(cp.y_col) + c0 * N + sb * kXS;
        const int m = t & 7;
        const uint32_t loff = (uint32_t)(t >> 3) * (uint32_t)N + 16u * (uint32_t)m;
#pragma unroll 4
        for (int it = 0; it < kXQ * 128 * 8 / ST; ++it) {
          const int qq = it >> 2, c32 = 32 * (it & 3);
          const uint4 v = *reinterpret_cast<const uint4 *>(stage[qq] + xstage(c32 + (t >> 3), 4 * m));
          st_nt16(cbase + (int64_t)(128 * qq + c32) * N + loff, v);
        }
      }
      if constexpr (MODE == MODE_MX) {
        // the super-band's 4 block exponents of each column: one 4-byte run
        uint8_t *const csb = static_cast<uint8_t *>(cp.col_scale_inv) + c0 * cp.mx_col_ld + 4 * sb;
#pragma unroll
        for (int h = 0; h < TW / ST; ++h) {
          const int col = t + ST * h;
          *reinterpret_cast<uint32_t *>(csb + (uint32_t)col * (uint32_t)cp.mx_col_ld) =
              *reinterpret_cast<const uint32_t *>(colx[col]);
        }
      }
    }
  };

  // step j: cur holds band j (its partials published two steps ago), sm holds band j + 2 (loaded
  // a step ago), ld receives band j + 3. Waves 0-1 poll band j while the others' loads go out; then
  // band j's codes and band j + 2's row sums; then waves 2-3 publish those sums and waves 4-7 write
  // band j's outputs. The row sums run on every step, also past the group's last band (on a tile
  // that was not loaded; nothing is published): every tile's loads are then waited for there, two
  // steps before its codes, on every path, so the compiler puts no wait for loads in flight into
  // the codes.
  auto step = [&](Tile &cur, Tile &sm, Tile &ld, int64_t j) {
    const bool do_ld = j + 3 < nb, do_sm = j + 2 < nb;
#pragma unroll
    for (int k = 0; k < KR; ++k) fresh<IN>(ld[k]);
    if (wave < kPollWaves) poll(j);
    else if (do_ld) load_tile(ld, j + 3);
    __syncthreads();
    if (wave < kPollWaves && do_ld) load_tile(ld, j + 3);
    codes(cur, j);
    row_sums(sm);
    __syncthreads();
    if (do_sm) publish(j + 2);
    if (wave >= kStoreWave0) store(j);
  };

  Tile T0, T1, T2, T3;
  if (nb > 0) {  // (nb is even: two bands per super-band)
#pragma unroll
    for (int k = 0; k < KR; ++k) fresh<IN>(T2[k]);
    load_tile(T0, 0);
    load_tile(T1, 1);
    if (nb > 2) load_tile(T2, 2);
    row_sums(T0);
    __syncthreads();
    publish(0);
    __syncthreads();
    row_sums(T1);
    __syncthreads();
    publish(1);
    __syncthreads();  // (the first step's sums rewrite rpart)
  }
  for (int64_t j = 0; j < nb; j += 4) {
    step(T0, T2, T3, j);
    if (j + 1 >= nb) break;
    step(T1, T3, T0, j + 1);
    if (j + 2 >= nb) break;
    step(T2, T0, T1, j + 2);
    if (j + 3 >= nb) break;
    step(T3, T1, T2, j + 3);
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

template <class IN, int FMT>
static const void *pick_colx_mode(int mode) {
  switch (mode) {
    case MODE_DELAYED: return (const void *)fwd_colx_kernel<IN, MODE_DELAYED, FMT>;
    case MODE_MX: return (const void *)fwd_colx_kernel<IN, MODE_MX, FMT>;
    default: return nullptr;
  }
}

template <class IN>
static const void *pick_colx_fmt(int out_dtype, int mode) {
  switch (out_dtype) {
    case DT_E4M3: return pick_colx_mode<IN, DT_E4M3>(mode);
    case DT_E5M2: return pick_colx_mode<IN, DT_E5M2>(mode);
    default: return nullptr;
  }
}

const void *fwd_colx_kernel_ptr(int in_dtype, int out_dtype, int mode) {
  switch (in_dtype) {
    // (float32 input: four bands would fill the registers; the two-pass routes serve it)
    case DT_BF16: return pick_colx_fmt<BF16>(out_dtype, mode);
    case DT_F16: return pick_colx_fmt<F16>(out_dtype, mode);
    default: return nullptr;
  }
}

}  // namespace nf8
