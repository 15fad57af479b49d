// fwd_band.hip -- LayerNorm / RMSNorm forward over tiles of several rows, for columnwise
// (transposed) FP8 outputs and for rows too long for one workgroup.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization";
// [NVRTC-PR] = "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request).
// [XLA-Norm] Description: rowwise and optional columnwise FP8 outputs, each with its own
// scale_inv, for delayed tensor scaling and MXFP8 block scaling. [NVRTC-PR] Flowchart and
// review discussion: rows too long for one CTA are split over several CTAs that combine their
// statistics through a workspace and a barrier.
//
// Work split: a workgroup (4 waves) owns a tile of R = 4 * RW rows x CW = 512 * KC columns;
// wave w owns rows [w*RW, (w+1)*RW) of the tile and lane l the strips l + 64k. S workgroups
// cover one band of R full rows. Each keeps its tile in registers (x is read from HBM once),
// computes per-row partial statistics, publishes them in the workspace and waits for the other
// S - 1 workgroups of its band; every workgroup then merges the S partials in slice order, so
// all S hold bit-identical statistics.
//
// Tiles are handed out in ticket order from an atomic counter, and a workgroup takes its next
// ticket only after it has stopped waiting on its current band. So a workgroup never holds a
// ticket of a band it is waiting on, every ticket holder is running, and at any time only the
// newest band can be waiting for a member whose ticket has not been taken yet: with at least
// 2S workgroups per ticket class some workgroup is always free to take it. No assumption about
// how many workgroups are resident is needed.
//
// Columnwise outputs: y_col is [hidden, rows]. MXFP8 columnwise blocks are the 32 rows of one
// band (RW = 8): each lane takes the max over its 8 rows per column, the 4 waves combine
// through LDS, and every lane writes its 8 rows of each column as one 8-byte store after an
// in-register byte transpose.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nf8 {

// 4x4 byte transpose of (a0..a3): result i holds byte i of a0, a1, a2, a3
__device__ __forceinline__ void transpose4x4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
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

// codes[j] = 8 codes of row j (columns 0..7); write column i's RW codes to colp + i * ld
template <int RW>
__device__ __forceinline__ void store_col_codes(const uint2 (&codes)[RW], uint8_t *colp, int64_t ld,
                                                int valid_rows, bool aligned) {
  static_assert(RW == 4 || RW == 8, "columnwise tiles hold 4 or 8 rows per wave");
  uint32_t lo[RW == 8 ? 2 : 1][4], hi[RW == 8 ? 2 : 1][4];
#pragma unroll
  for (int h = 0; h < RW / 4; ++h) {
    transpose4x4(codes[4 * h].x, codes[4 * h + 1].x, codes[4 * h + 2].x, codes[4 * h + 3].x, lo[h]);
    transpose4x4(codes[4 * h].y, codes[4 * h + 1].y, codes[4 * h + 2].y, codes[4 * h + 3].y, hi[h]);
  }
  if (aligned && valid_rows == RW) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint8_t *dst = colp + i * ld;
      const uint32_t w0 = i < 4 ? lo[0][i] : hi[0][i - 4];
      if constexpr (RW == 8) {
        const uint32_t w1 = i < 4 ? lo[1][i] : hi[1][i - 4];
        st_nt8(dst, make_uint2(w0, w1));
      } else {
        *reinterpret_cast<uint32_t *>(dst) = w0;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint8_t *dst = colp + i * ld;
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const uint32_t w = i < 4 ? lo[j / 4][i] : hi[j / 4][i - 4];
        if (j < valid_rows) dst[j] = (uint8_t)(w >> (8 * (j & 3)));
      }
    }
  }
}

template <int NORM, class IN, int MODE, int RW, int KC, bool COL>
__global__ __launch_bounds__(256) void fwd_band_kernel(FwdBandParams bp) {
  constexpr int R = 4 * RW;
  constexpr int CW = 512 * KC;
  constexpr bool MXCOL = COL && MODE == MODE_MX;
  const FwdRowParams &p = bp.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int S = bp.S;
  const int64_t H = p.hidden;
  const int64_t N = p.rows;
  const int fmt = p.out_dtype;

  constexpr int NV = NORM == NT_LAYERNORM ? 3 : 1;  // tagged words per row partial (mean, M2, shift)
  __shared__ int64_t s_next;
  __shared__ uint32_t s_last;
  __shared__ uint32_t s_epoch;
  __shared__ float wred[4];
  __shared__ float colmax[MXCOL ? 4 : 1][MXCOL ? CW : 1];
  __shared__ float xpart[4][RW][kMaxSlices][NV];  // fetched partials of the band's rows

  // Ticket class: the workgroups with the same blockIdx % classes serve one contiguous range
  // of bands. Consecutive workgroups are dispatched to the XCDs in turn, so a class's bands --
  // and the columnwise segments that neighbouring bands write into the same cache lines --
  // stay within one L2.
  const int ncls = bp.classes;
  const int cls = (int)(blockIdx.x % ncls);
  const int64_t wpc = gridDim.x / ncls;
  const int64_t lwg = blockIdx.x / ncls;
  const int64_t b0 = bp.bands * cls / ncls;
  const int64_t b1 = bp.bands * (cls + 1) / ncls;
  const int64_t ntiles = (b1 - b0) * S;
  uint32_t *const ticket = S > 1 ? p.ws + kWsTicket0 + cls : nullptr;
  const bool coordinated = MODE == MODE_DELAYED || S > 1;
  const uint32_t tag = coordinated ? epoch_tag(read_epoch(p.ws, &s_epoch)) : 0u;

  int64_t tk;
  if (S == 1) {
    tk = lwg;
  } else {
    if (tid == 0) s_next = (int64_t)add_dev(ticket, 1u);
    __syncthreads();
    tk = s_next;
    __syncthreads();
  }

  float scale = 1.0f;
  if constexpr (MODE == MODE_DELAYED) scale = *p.scale;
  float amax_local = 0.0f;
  const float inv_h = 1.0f / (float)H;
  const bool col_aligned = (N % RW) == 0;

  while (tk < ntiles) {
    const int64_t lband = tk / S;
    const int64_t band = b0 + lband;
    const int slice = (int)(tk - lband * S);
    const int64_t rbase = band * R + wave * RW;  // first row of this wave
    const int64_t cbase = (int64_t)slice * CW;

    // Weights are read per strip where they are used (they stay in L1/L2 for the tile's rows)
    // instead of being held in registers for every strip of the tile.
    bool cv[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) cv[k] = cbase + 8 * (lane + 64 * k) < H;
    auto weights = [&](int k, float (&g)[8], float (&bt)[8]) {
      const int64_t col = cbase + 8 * (lane + 64 * k);
      if (cv[k]) {
        load_w8(g, p.gamma, col, p.w_dtype);
        if (p.zero_centered) {
#pragma unroll
          for (int i = 0; i < 8; ++i) g[i] += 1.0f;
        }
        if constexpr (NORM == NT_LAYERNORM) load_w8(bt, p.beta, col, p.w_dtype);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          g[i] = 0.0f;
          bt[i] = 0.0f;
        }
      }
    };

    Strip<IN> xs[RW][KC];
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int64_t row = rbase + j;
        if (row < N && cv[k]) load_strip<IN>(xs[j][k], p.x, row * H + cbase + 8 * (lane + 64 * k));
        else zero_strip<IN>(xs[j][k]);
      }

    // ---- per-row partial statistics of this slice (wave-merged). LayerNorm: taken relative
    // to a shift K near the mean -- the slice's plain mean estimate of the row -- so that a row
    // with a large common part keeps its deviations
    Stats st[RW];
    float shift[RW];
    const float inv_ns = 1.0f / (float)(H - cbase < CW ? H - cbase : CW);  // this slice's columns
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      const bool rv = rbase + j < N;
      shift[j] = 0.0f;
      if constexpr (NORM == NT_LAYERNORM) {
        {
          float sa = 0.0f;
#pragma unroll
          for (int k = 0; k < KC; ++k) {
            float xv[8];
            strip_to_f32<IN>(xs[j][k], xv);
#pragma unroll
            for (int i = 0; i < 8; ++i) sa += xv[i];  // (strips outside the tensor are zero)
          }
          shift[j] = first_lane(wave_sum(sa) * inv_ns);  // rounded once (no fma fusion into x - K)
        }
        float sm = 0.0f, n = 0.0f;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          float xv[8];
          strip_to_f32<IN>(xs[j][k], xv);
          if (rv && cv[k]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) sm += xv[i] - shift[j];
            n += 8.0f;
          }
        }
        const float m = n > 0.0f ? sm / n : 0.0f;
        float q = 0.0f;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          float xv[8];
          strip_to_f32<IN>(xs[j][k], xv);
          if (rv && cv[k]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float d = (xv[i] - shift[j]) - m;
              q = fmaf(d, d, q);
            }
          }
        }
        st[j] = wave_merge(Stats{n, m, q});
      } else {
        float q = 0.0f;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          float xv[8];
          strip_to_f32<IN>(xs[j][k], xv);
#pragma unroll
          for (int i = 0; i < 8; ++i) q = fmaf(xv[i], xv[i], q);
        }
        st[j] = Stats{0.0f, 0.0f, wave_sum(q)};
      }
    }

    // ---- combine the S slices of the band through the workspace: publish this slice's
    // tagged row partials, then every lane polls one (row, slice, word) of the band until it
    // carries this launch's tag; lane j merges row j's S partials in slice order from LDS and
    // broadcasts the result to the wave
    if (S > 1) {
      uint64_t *part = bp.partials + (band * S + slice) * (int64_t)R * NV;
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        if (lane == j) {
          if constexpr (NORM == NT_LAYERNORM) {
            st_dev64(part + (wave * RW + j) * NV, tagged(st[j].mean, tag));
            st_dev64(part + (wave * RW + j) * NV + 1, tagged(st[j].m2, tag));
            st_dev64(part + (wave * RW + j) * NV + 2, tagged(shift[j], tag));
          } else {
            st_dev64(part + (wave * RW + j), tagged(st[j].m2, tag));
          }
        }
      }
      const uint64_t *bpart = bp.partials + band * S * (int64_t)R * NV;
      for (int l = lane; l < RW * S * NV; l += 64) {
        const int v = l % NV, js = l / NV;
        const int j = js / S, sl = js - (js / S) * S;
        xpart[wave][j][sl][v] = wait_tagged(bpart + ((int64_t)sl * R + wave * RW + j) * NV + v, tag, p.ws + kWsError);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        Stats acc{0.0f, 0.0f, 0.0f};
        float k0 = 0.0f;
        if (lane == j) {
          if constexpr (NORM == NT_LAYERNORM) k0 = xpart[wave][j][0][2];  // slice 0's frame
          for (int sl = 0; sl < S; ++sl) {
            if constexpr (NORM == NT_LAYERNORM) {
              const int64_t left = H - (int64_t)sl * CW;
              const float n = (float)(left < CW ? left : CW);
              const ShiftedStats o{Stats{n, xpart[wave][j][sl][0], xpart[wave][j][sl][1]}, xpart[wave][j][sl][2]};
              acc = chan_merge(acc, in_frame(o, k0));
            } else {
              acc.m2 += xpart[wave][j][sl][0];
            }
          }
        }
        st[j].mean = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acc.mean), j));
        st[j].m2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acc.m2), j));
        shift[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, k0), j));
      }
    }
    // The next tile's ticket is taken only now, once this workgroup waits for nothing more in
    // its current band (a ticket taken earlier could be a slice of the band it is waiting on,
    // which it could then never deliver); its latency overlaps the output phase.
    if (S > 1 && tid == 0) s_next = (int64_t)add_dev(ticket, 1u);

    float mu[RW], rs[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      mu[j] = NORM == NT_LAYERNORM ? shift[j] + st[j].mean : 0.0f;
      rs[j] = 1.0f / sqrtf(st[j].m2 * inv_h + p.eps);
      const int64_t row = rbase + j;
      if (slice == 0 && lane == j && row < N) {
        if (p.rsigma) p.rsigma[row] = rs[j];
        if constexpr (NORM == NT_LAYERNORM) {
          if (p.mu) p.mu[row] = mu[j];
        }
      }
    }
    const int valid_rows = (int)(N - rbase < RW ? (N - rbase < 0 ? 0 : N - rbase) : RW);

    // ---- MXFP8 columnwise block maxima (32 rows = the 4 waves' rows of this band)
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
      for (int k = 0; k < KC; ++k) opaque<IN>(xs[j][k]);
    if constexpr (MXCOL) {
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float cm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        float gk[8], bk[8];
        weights(k, gk, bk);
#pragma unroll
        for (int j = 0; j < RW; ++j) {
          float xv[8];
          strip_to_f32<IN>(xs[j][k], xv);
          if (j < valid_rows) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              float y;
              if constexpr (NORM == NT_LAYERNORM) y = fmaf((xv[i] - mu[j]) * rs[j], gk[i], bk[i]);
              else y = (xv[i] * rs[j]) * gk[i];
              cm[i] = fmaxf(cm[i], fabsf(y));
            }
          }
        }
        float4 *dst = reinterpret_cast<float4 *>(&colmax[wave][8 * (lane + 64 * k)]);
        dst[0] = make_float4(cm[0], cm[1], cm[2], cm[3]);
        dst[1] = make_float4(cm[4], cm[5], cm[6], cm[7]);
      }
      __syncthreads();
    }

    // ---- outputs, one strip column at a time
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
      for (int k = 0; k < KC; ++k) opaque<IN>(xs[j][k]);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int64_t col = cbase + 8 * (lane + 64 * k);
      float gk[8], bk[8];
      weights(k, gk, bk);
      uint2 rcodes[RW];  // rowwise codes (delayed: reused for the columnwise transpose)
      float colf[8];     // MX columnwise: 2^-X per column
      int colx[8];
      if constexpr (MXCOL) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = 8 * (lane + 64 * k) + i;
          const float a = fmaxf(fmaxf(colmax[0][c], colmax[1][c]), fmaxf(colmax[2][c], colmax[3][c]));
          colx[i] = mx_exponent(a, fmt, p.mx_ceil);
          colf[i] = exp2_neg(colx[i]);
        }
      }
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const int64_t row = rbase + j;
        const bool ok = (j < valid_rows) && cv[k];
        float xv[8], y[8];
        strip_to_f32<IN>(xs[j][k], xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if constexpr (NORM == NT_LAYERNORM) y[i] = fmaf((xv[i] - mu[j]) * rs[j], gk[i], bk[i]);
          else y[i] = (xv[i] * rs[j]) * gk[i];
        }
        if constexpr (MODE == MODE_PLAIN) {
          if (ok) store_out8(p.y, row * H + col, y, p.out_dtype);
        } else if constexpr (MODE == MODE_DELAYED) {
          float u[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            u[i] = y[i] * scale;
            if (ok) amax_local = fmaxf(amax_local, fabsf(y[i]));
          }
          rcodes[j] = fp8_pack8(u, fmt);
          if (ok && bp.write_row)
            st_nt8(static_cast<uint8_t *>(p.y) + row * H + col, rcodes[j]);
        } else {  // MX
          if (bp.write_row) {
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(y[i]));
            a = quad_max(ok ? a : 0.0f);
            const int X = mx_exponent(a, fmt, p.mx_ceil);
            const float f = exp2_neg(X);
            float u[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = y[i] * f;
            const uint2 c = fp8_pack8(u, fmt);
            if (ok) {
              st_nt8(static_cast<uint8_t *>(p.y) + row * H + col, c);
              if ((lane & 3) == 0)
                static_cast<uint8_t *>(p.scale_inv)[row * p.mx_cols + (col >> 5)] = (uint8_t)(X + 127);
            }
          }
          if constexpr (MXCOL) {
            float u[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = y[i] * colf[i];
            rcodes[j] = fp8_pack8(u, fmt);
          }
        }
      }
      if constexpr (COL && MODE != MODE_PLAIN) {
        if (cv[k] && valid_rows > 0) {
          uint8_t *colp = static_cast<uint8_t *>(bp.y_col) + col * N + rbase;
          store_col_codes<RW>(rcodes, colp, N, valid_rows, col_aligned);
          if constexpr (MXCOL) {
            if (wave == 0) {
#pragma unroll
              for (int i = 0; i < 8; ++i)
                static_cast<uint8_t *>(bp.col_scale_inv)[(col + i) * bp.mx_col_ld + band] = (uint8_t)(colx[i] + 127);
            }
          }
        }
      }
    }
    __syncthreads();  // LDS (colmax, xpart) is reused by the next tile; s_next is visible
    tk = S > 1 ? s_next : tk + wpc;
  }

  // ---- end of launch: amax publication and counter reset by the last workgroup
  if constexpr (MODE == MODE_DELAYED) {
    const float m = wave_max(amax_local);
    if (lane == 0) wred[wave] = m;
    __syncthreads();
    if (tid == 0) {
      publish_amax(p.ws, fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3])), tag);
      if (blockIdx.x == 0) {
        if (p.scale_inv) *static_cast<float *>(p.scale_inv) = 1.0f / scale;
        if (bp.col_scale_inv) *static_cast<float *>(bp.col_scale_inv) = 1.0f / scale;
      }
    }
  }
  if (coordinated) {
    vmem_drain();
    if (finish_workgroup(p.ws, &s_last)) {
      if constexpr (MODE == MODE_DELAYED) {
        __syncthreads();
        const float tot = gather_amax(p.ws, gridDim.x, wred, tag);
        if (tid == 0) *p.updated_amax = fmaxf(*p.amax_in, tot);
      }
      if (S > 1 && tid < ncls) xchg_dev(p.ws + kWsTicket0 + tid, 0u);
      vmem_drain();
      __syncthreads();
      reset_completion(p.ws);
    }
  }
}

// ------------------------------------------------------------------------------------------

template <int NORM, class IN, int MODE, bool COL>
static const void *pick_band_cfg(int cfg) {
  switch (cfg) {
    case BAND_R8_K1: return (const void *)fwd_band_kernel<NORM, IN, MODE, 8, 1, COL>;
    case BAND_R8_K2: return (const void *)fwd_band_kernel<NORM, IN, MODE, 8, 2, COL>;
    case BAND_R4_K2:
      if constexpr (COL && MODE == MODE_MX) return nullptr;  // MX columnwise blocks need 32-row bands
      else return (const void *)fwd_band_kernel<NORM, IN, MODE, 4, 2, COL>;
    case BAND_R1_K4: return COL ? nullptr : (const void *)fwd_band_kernel<NORM, IN, MODE, 1, 4, false>;
    case BAND_R2_K8: return COL ? nullptr : (const void *)fwd_band_kernel<NORM, IN, MODE, 2, 8, false>;
    default: return nullptr;
  }
}

template <int NORM, class IN>
static const void *pick_band_mode(int mode, bool col, int cfg) {
  switch (mode) {
    case MODE_PLAIN: return col ? nullptr : pick_band_cfg<NORM, IN, MODE_PLAIN, false>(cfg);
    case MODE_DELAYED:
      return col ? pick_band_cfg<NORM, IN, MODE_DELAYED, true>(cfg)
                 : pick_band_cfg<NORM, IN, MODE_DELAYED, false>(cfg);
    case MODE_MX:
      return col ? pick_band_cfg<NORM, IN, MODE_MX, true>(cfg) : pick_band_cfg<NORM, IN, MODE_MX, false>(cfg);
    default: return nullptr;
  }
}

template <int NORM>
static const void *pick_band_in(int in_dtype, int mode, bool col, int cfg) {
  switch (in_dtype) {
    case DT_F32: return pick_band_mode<NORM, F32>(mode, col, cfg);
    case DT_BF16: return pick_band_mode<NORM, BF16>(mode, col, cfg);
    case DT_F16: return pick_band_mode<NORM, F16>(mode, col, cfg);
    default: return nullptr;
  }
}

const void *fwd_band_kernel_ptr(int norm, int in_dtype, int mode, bool col, int cfg) {
  return norm == NT_LAYERNORM ? pick_band_in<NT_LAYERNORM>(in_dtype, mode, col, cfg)
                              : pick_band_in<NT_RMSNORM>(in_dtype, mode, col, cfg);
}

}  // namespace nf8
