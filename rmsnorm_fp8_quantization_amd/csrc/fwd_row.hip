// fwd_row.hip -- LayerNorm / RMSNorm forward with a fused output epilogue, one row per team.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization".
// [XLA-Norm] Overview / Description: LayerNorm or RMSNorm forward that writes the normalised
// output (optionally FP8-quantised with delayed per-tensor or MXFP8 block scaling, in the
// same kernel launch) plus mu (LayerNorm) and rsigma for the backward. MODE_STATS writes only
// mu / rsigma (the first pass of the columnwise path, see fwd_col.hip). [XLA-Norm] I/O Contract
// lists the inputs (x, gamma, beta, scale, amax) and outputs (y, mu, rsigma, scale_inv,
// updated amax) this kernel reads and writes.
//
// Work split: a team of P waves owns one row at a time (P = 1: a wave per row; P > 1: the
// waves exchange partial statistics through LDS). A workgroup holds T teams and walks over
// rows with a grid stride, keeping gamma / beta in registers across rows. Each lane owns KC
// strips of 8 consecutive elements, so a row of up to 512 * P * KC elements is read from HBM
// exactly once into registers; statistics, normalisation and the epilogue run on the
// registers.
//
// Statistics: each lane reduces its own strips exactly (local mean, then local sum of squared
// deviations, or the sum of squares for RMSNorm), lanes merge with DPP/swizzle steps and the
// parallel-variance (Chan) merge, waves merge through LDS in a fixed order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nf8 {

// weight lookahead of the long-row layout, in strips (2 spills registers)
constexpr int kWeightLookahead = 1;

// WL: where the weights live while the workgroup walks its rows. 0: each lane keeps its
// columns' gamma / beta in registers; 1: the workgroup stages them once in LDS (as float32,
// 1 + gamma when zero-centred), leaving the registers to the row data so that the next row
// can be in flight while the current one is normalised; 2 (rows too long for either): each
// strip's weights are read where they are used (they stay in the L2 across rows).
template <int NORM, class IN, int MODE, int P, int T, int KC, int WL>
__global__ __launch_bounds__(64 * P * T) void fwd_row_kernel(FwdRowParams p) {
  constexpr int TEAM = 64 * P;
  constexpr int NT = TEAM * T;
  constexpr int COVER = 8 * TEAM * KC;                      // row elements one team holds
  constexpr int NW = NORM == NT_LAYERNORM ? 2 : 1;          // weight arrays
  // many strips per lane: convert them again for each pass instead of keeping 8 KC floats
  // live, which would leave no room for the next row's loads
  constexpr bool RECONV = WL == 2 || KC >= 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int team = wave / P;
  const int wt = wave - team * P;
  const int tl = tid - team * TEAM;
  const int64_t H = p.hidden;
  const int fmt = p.out_dtype;

  bool cv[KC];
  float n_in = 0.0f;  // this lane's elements inside the row
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    cv[k] = 8 * (int64_t)(tl + TEAM * k) < H;
    n_in += cv[k] ? 8.0f : 0.0f;
  }

  // ---- weights
  __shared__ float wlds[WL == 1 && MODE != MODE_STATS ? NW * COVER : 1];  // (statistics: no weights)
  float g[WL ? 1 : KC][8];
  float b[(!WL && NORM == NT_LAYERNORM) ? KC : 1][8];
  if constexpr (WL == 2 || MODE == MODE_STATS) {
    // nothing staged
  } else if constexpr (WL == 1) {
    for (int64_t c = 8 * (int64_t)tid; c < H; c += 8 * NT) {
      float w[8];
      load_w8(w, p.gamma, c, p.w_dtype);
      if (p.zero_centered) {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] += 1.0f;
      }
      float4 *d = reinterpret_cast<float4 *>(wlds + c);
      d[0] = make_float4(w[0], w[1], w[2], w[3]);
      d[1] = make_float4(w[4], w[5], w[6], w[7]);
      if constexpr (NORM == NT_LAYERNORM) {
        load_w8(w, p.beta, c, p.w_dtype);
        float4 *e = reinterpret_cast<float4 *>(wlds + COVER + c);
        e[0] = make_float4(w[0], w[1], w[2], w[3]);
        e[1] = make_float4(w[4], w[5], w[6], w[7]);
      }
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int64_t col = 8 * (int64_t)(tl + TEAM * k);
      if (cv[k]) {
        load_w8(g[k], p.gamma, col, p.w_dtype);
        if (p.zero_centered) {
#pragma unroll
          for (int i = 0; i < 8; ++i) g[k][i] += 1.0f;
        }
        if constexpr (NORM == NT_LAYERNORM) load_w8(b[k], p.beta, col, p.w_dtype);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          g[k][i] = 0.0f;
          if constexpr (NORM == NT_LAYERNORM) b[k][i] = 0.0f;
        }
      }
    }
  }
  // WL == 2: strip k's raw weights are loaded ahead of their use and converted where used
  auto weights_raw = [&](int k, W8Raw &rg, W8Raw &rb) {
    uint32_t c = cv[k] ? 8u * (uint32_t)(tl + TEAM * k) : 0u;
    // formed where it is used (a scalar base plus this 32-bit offset) rather than hoisted out
    // of the row loop as 64-bit addresses held for every strip
    asm volatile("" : "+v"(c));
    load_w8_raw(rg, p.gamma, c, p.w_dtype);
    if constexpr (NORM == NT_LAYERNORM) load_w8_raw(rb, p.beta, c, p.w_dtype);
  };
  auto weights_cvt = [&](int k, const W8Raw &rg, const W8Raw &rb, float (&gk)[8], float (&bk)[8]) {
    w8_convert(gk, rg, p.w_dtype);
    if constexpr (NORM == NT_LAYERNORM) w8_convert(bk, rb, p.w_dtype);
    const float z = p.zero_centered ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // strips past the end read column 0: zero them
      gk[i] = cv[k] ? gk[i] + z : 0.0f;
      if constexpr (NORM == NT_LAYERNORM) bk[i] = cv[k] ? bk[i] : 0.0f;
    }
  };
  // the 8 weights of strip k (from the caches, LDS or registers)
  auto weights = [&](int k, float (&gk)[8], float (&bk)[8]) {
    if constexpr (WL == 2) {
      W8Raw rg, rb;
      weights_raw(k, rg, rb);
      weights_cvt(k, rg, rb, gk, bk);
    } else if constexpr (WL == 1) {
      const int c = 8 * (tl + TEAM * k);
      const float4 *s0 = reinterpret_cast<const float4 *>(wlds + c);
      float4 a = s0[0], d = s0[1];
      gk[0] = a.x; gk[1] = a.y; gk[2] = a.z; gk[3] = a.w; gk[4] = d.x; gk[5] = d.y; gk[6] = d.z; gk[7] = d.w;
      if constexpr (NORM == NT_LAYERNORM) {
        const float4 *s1 = reinterpret_cast<const float4 *>(wlds + COVER + c);
        a = s1[0];
        d = s1[1];
        bk[0] = a.x; bk[1] = a.y; bk[2] = a.z; bk[3] = a.w; bk[4] = d.x; bk[5] = d.y; bk[6] = d.z; bk[7] = d.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        gk[i] = g[k][i];
        if constexpr (NORM == NT_LAYERNORM) bk[i] = b[k][i];
      }
    }
  };

  float scale = 1.0f;
  // launch epoch (thread 0): loaded here, first needed when the workgroup publishes its amax,
  // so nothing waits for it before the first row's loads go out
  uint32_t epoch = 0;
  __shared__ uint32_t s_epoch;
  if constexpr (MODE == MODE_DELAYED) {
    scale = *p.scale;
    if (tid == 0) epoch = ld_dev_u32(p.ws + kWsEpoch);
  }
  float amax_local = 0.0f;

  __shared__ ShiftedStats red[2][T][P];
  const float inv_h = 1.0f / (float)H;
  // reciprocal of the number of row elements this wave holds (LayerNorm's shift estimate)
  const float inv_nw = P == 1 ? inv_h : 1.0f / fmaxf(wave_sum(n_in), 1.0f);
  const int64_t stride = (int64_t)gridDim.x * T;

  // Loads are unconditional (rows past the end read row 0, strips past the end of the row read
  // column 0) and the strips are masked where they are used: a load under a branch may not have
  // been issued, so the wait before the current row's first use would have to drain the
  // prefetch of the next row as well.
  auto load_row = [&](Strip<IN> (&xs)[KC], int64_t row) {
    const int64_t r = row < p.rows ? row : 0;
#pragma unroll
    for (int k = 0; k < KC; ++k) load_strip<IN>(xs[k], p.x, r * H + (cv[k] ? 8 * (int64_t)(tl + TEAM * k) : 0));
  };

  // software pipeline: the next row's loads are issued before the current row is normalised
  // (not with WL == 2: the registers hold the weights in flight instead)
  constexpr bool PF = WL != 2;
  Strip<IN> cur[KC], nxt[PF ? KC : 1];
  int64_t base = (int64_t)blockIdx.x * T;
  load_row(cur, base + team);
  int iter = 0;
  for (; base < p.rows; base += stride, ++iter) {
    const int64_t row = base + team;
    const bool rv = row < p.rows;
    if constexpr (PF) load_row(nxt, base + stride + team);
    if (H != COVER) {  // strips past the end of the row read column 0: zero them
#pragma unroll
      for (int k = 0; k < KC; ++k) mask_strip<IN>(cur[k], cv[k]);
    }
    // WL == 2: the weights of strip k are loaded WLA strips ahead of their use (WLA + 1
    // buffers in turn); the first ones go out before the statistics so their latency hides
    // behind them
    constexpr int WLA = kWeightLookahead;
    constexpr int WQ = WL == 2 && MODE != MODE_STATS ? WLA + 1 : 1;
    W8Raw wq_g[WQ], wq_b[WQ];
    if constexpr (WQ > 1) {
#pragma unroll
      for (int k = 0; k < WLA && k < KC; ++k) weights_raw(k, wq_g[k], wq_b[k]);
    }

    // ---- lane-local statistics over its valid strips. LayerNorm takes every deviation from a
    // shift K near the mean -- the wave's plain mean estimate (sum of its elements over their
    // count) -- so that a row whose values share a large common part keeps its deviations, and
    // the mean comes out as K + (mean - K), rounded once; strips past the end add nothing.
    Stats st{0.0f, 0.0f, 0.0f};
    float shift = 0.0f;
    if constexpr (NORM == NT_LAYERNORM) {
      {
        float sa = 0.0f;
#pragma unroll
        for (int k = 0; k < KC; ++k) sa += strip_sum<IN>(cur[k]);  // (strips past the end are zero)
        // (through readfirstlane: the shift is rounded once and every use sees that value; a
        // product left in a register would be fused into each x - K as an fma, putting the
        // deviations in a frame of the unrounded product)
        shift = first_lane(wave_sum(sa) * inv_nw);
      }
      if constexpr (RECONV) {
#pragma unroll
        for (int k = 0; k < KC; ++k) opaque<IN>(cur[k]);
      }
      // one pass over the deviations d = x - K of the valid elements: their sum and sum of
      // squares. With K near the mean the lane's (and the row's) mean deviation is small
      // against the spread, so M2 = sum d^2 - (sum d)^2 / n loses nothing to cancellation.
      // Strip k is inside the row for every lane of the team when 8 * TEAM * (k + 1) <= H (a
      // uniform test); only other strips need the per-lane mask.
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xv[8];
        strip_to_f32<IN>(cur[k], xv);
        if (8 * (int64_t)TEAM * (k + 1) <= H) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float d = xv[i] - shift;
            s1 += d;
            s2 = fmaf(d, d, s2);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float d = cv[k] ? xv[i] - shift : 0.0f;
            s1 += d;
            s2 = fmaf(d, d, s2);
          }
        }
      }
      if constexpr (P == 1) {
        // one wave holds the row: its mean deviation and M2 directly
        const float t1 = wave_sum(s1), t2 = wave_sum(s2);
        const float m = t1 * inv_h;
        st = Stats{(float)H, m, fmaxf(fmaf(-t1, m, t2), 0.0f)};
      } else {
        // several waves: per-lane (n, mean, M2), merged in the Chan form
        const float m = n_in > 0.0f ? s1 * __builtin_amdgcn_rcpf(n_in) : 0.0f;
        st = wave_merge(Stats{n_in, m, fmaxf(fmaf(-s1, m, s2), 0.0f)});
      }
    } else {
      float q = 0.0f;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xv[8];
        strip_to_f32<IN>(cur[k], xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) q = fmaf(xv[i], xv[i], q);  // masked strips are zero
      }
      st.m2 = wave_sum(q);
    }

    // ---- merge the team's waves in a fixed order (LayerNorm: each wave's partial moved into
    // wave 0's frame)
    if constexpr (P > 1) {
      if (lane == 0) red[iter & 1][team][wt] = ShiftedStats{st, shift};
      __syncthreads();
      st = red[iter & 1][team][0].s;
      shift = red[iter & 1][team][0].k;
#pragma unroll
      for (int w = 1; w < P; ++w) {
        const ShiftedStats o = red[iter & 1][team][w];
        if constexpr (NORM == NT_LAYERNORM) st = chan_merge(st, in_frame(o, shift));
        else st.m2 += o.s.m2;
      }
    }

    const float mu = NORM == NT_LAYERNORM ? shift + st.mean : 0.0f;
    const float rs = __builtin_amdgcn_rsqf(st.m2 * inv_h + p.eps);
    if constexpr (RECONV) {
#pragma unroll
      for (int k = 0; k < KC; ++k) opaque<IN>(cur[k]);
    }
    if (rv && tl == 0) {
      if (p.rsigma) p.rsigma[row] = rs;
      if constexpr (NORM == NT_LAYERNORM) {
        if (p.mu) p.mu[row] = mu;
      }
    }

    // ---- normalise and store (WL == 2: a scheduling barrier per strip keeps one strip's
    // weights live at a time)
#pragma unroll
    for (int k = 0; k < (MODE == MODE_STATS ? 0 : KC); ++k) {
      // FP8 output, four or more strips per lane: a strip that lies past the row's end for the
      // whole team is skipped (no weights, arithmetic or store; with MXFP8 no lane of any of its
      // blocks is inside the row). The test is the same for every lane of the team, so its
      // waves stay balanced; skipping per lane, where only some waves of a team are past the
      // end, gained nothing. The branch itself costs a few percent where it never skips, so
      // layouts of fewer strips, which rarely have a whole strip past the end, go without it,
      // and so does plain output, which measured the same either way. (WL == 2 loads later
      // strips' weights in this pass.)
      if constexpr (WL != 2 && (MODE == MODE_DELAYED || MODE == MODE_MX) && KC >= 4) {
        if (8 * (int64_t)TEAM * k >= H) continue;
      }
      const bool ok = rv && cv[k];
      const int64_t col = 8 * (int64_t)(tl + TEAM * k);
      float gk[8], bk[8], xv[8], y[8];
      if constexpr (WQ > 1) {
        if (k + WLA < KC) weights_raw(k + WLA, wq_g[(k + WLA) % WQ], wq_b[(k + WLA) % WQ]);
        weights_cvt(k, wq_g[k % WQ], wq_b[k % WQ], gk, bk);
      } else {
        weights(k, gk, bk);
      }
      strip_to_f32<IN>(cur[k], xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (NORM == NT_LAYERNORM) y[i] = fmaf((xv[i] - mu) * rs, gk[i], bk[i]);
        else y[i] = (xv[i] * rs) * gk[i];
      }
      if constexpr (MODE == MODE_PLAIN) {
        if (ok) store_out8(p.y, row * H + col, y, fmt);
      } else if constexpr (MODE == MODE_DELAYED) {
        float u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          u[i] = y[i] * scale;
          if (ok) amax_local = fmaxf(amax_local, fabsf(y[i]));
        }
        const uint2 c = fp8_pack8(u, fmt);
        if (ok) st_nt8(static_cast<uint8_t *>(p.y) + row * H + col, c);
      } else {  // MODE_MX: 4 consecutive lanes hold one 32-element block
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
          if ((tl & 3) == 0)
            static_cast<uint8_t *>(p.scale_inv)[row * p.mx_cols + (col >> 5)] = (uint8_t)(X + 127);
        }
      }
      if constexpr (WL == 2) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (PF) {
#pragma unroll
      for (int k = 0; k < KC; ++k) cur[k] = nxt[k];
    } else {
      // (loads return in issue order: the next row's loads go out after the last weight load
      // this row needs, or every weight load behind them would wait for HBM)
      load_row(cur, base + stride + team);
    }
  }

  if constexpr (MODE == MODE_DELAYED) {
    // tensor amax: workgroup max -> this workgroup's tagged slot; the last workgroup to finish
    // takes the max over all slots, publishes max(amax_in, amax) and re-zeroes the counters
    __shared__ float wred[P * T];
    __shared__ uint32_t last_flag;
    const float m = wave_max(amax_local);
    if (lane == 0) wred[wave] = m;
    __syncthreads();
    if (tid == 0) {
      float a = wred[0];
#pragma unroll
      for (int w = 1; w < P * T; ++w) a = fmaxf(a, wred[w]);
      s_epoch = epoch;  // for the last workgroup's gather (visible after finish_workgroup's barrier)
      publish_amax(p.ws, a, epoch_tag(epoch));
      if (blockIdx.x == 0) *static_cast<float *>(p.scale_inv) = 1.0f / scale;
    }
    vmem_drain();
    if (finish_workgroup(p.ws, &last_flag)) {
      const float tot = gather_amax(p.ws, gridDim.x, wred, epoch_tag(s_epoch));
      if (tid == 0) *p.updated_amax = fmaxf(*p.amax_in, tot);
      reset_completion(p.ws);
    }
  }
}

// ------------------------------------------------------------------------------------------
// instantiation table
// ------------------------------------------------------------------------------------------

// weights go to LDS when the team's cover of float32 gamma (and beta) fits in 64 KB; with 8
// strips per lane and a larger cover they are read per strip from the caches
template <int NORM, int P, int KC> constexpr int wl_for() {
  return (NORM == NT_LAYERNORM ? 2 : 1) * 8 * 64 * P * KC * 4 <= 65536 && KC >= 4 ? 1 : (KC >= 8 ? 2 : 0);
}

template <int NORM, class IN, int MODE>
static const void *pick_cfg(int cfg) {
#define NF8_ROW(P, T, KC) (const void *)fwd_row_kernel<NORM, IN, MODE, P, T, KC, wl_for<NORM, P, KC>()>
  switch (cfg) {
    case ROW_W1_K1: return NF8_ROW(1, 4, 1);
    case ROW_W1_K2: return NF8_ROW(1, 4, 2);
    case ROW_W1_K4: return NF8_ROW(1, 4, 4);
    case ROW_W1_K8: return NF8_ROW(1, 4, 8);
    case ROW_W4_K2: return NF8_ROW(4, 1, 2);
    case ROW_W4_K4: return NF8_ROW(4, 1, 4);
    case ROW_W8_K4: return NF8_ROW(8, 1, 4);
    case ROW_W2T2_K4: return NF8_ROW(2, 2, 4);
    case ROW_W8_K1: return NF8_ROW(8, 1, 1);
    case ROW_W4T2_K2: return NF8_ROW(4, 2, 2);
    case ROW_W16_K8: return NF8_ROW(16, 1, 8);
    case ROW_W4T4_K4: return NF8_ROW(4, 4, 4);
    case ROW_W16_K2: return NF8_ROW(16, 1, 2);
    // weights in LDS whatever their size (LayerNorm: 128 KB for 16384 elements, one workgroup
    // of 16 waves per CU)
    case ROW_W8T2_K4: return (const void *)fwd_row_kernel<NORM, IN, MODE, 8, 2, 4, 1>;
    // RMSNorm: gamma in registers (32 per lane, loaded once per persistent workgroup);
    // LayerNorm's gamma and beta would need 64 and spill, so they are read per strip
    case ROW_W16_K4:
      return (const void *)fwd_row_kernel<NORM, IN, MODE, 16, 1, 4, NORM == NT_LAYERNORM ? 2 : 0>;
    // weights in registers for the whole persistent workgroup (LayerNorm: 128 per lane, 244-248
    // VGPRs); the FP8 epilogues and float32 input would spill there
    case ROW_W8_K8:
      if constexpr ((MODE == MODE_PLAIN || MODE == MODE_STATS) && IN::bytes == 2)
        return (const void *)fwd_row_kernel<NORM, IN, MODE, 8, 1, 8, 0>;
      return nullptr;
    case ROW_W4_K8:
      if constexpr ((MODE == MODE_PLAIN || MODE == MODE_STATS) && IN::bytes == 2)
        return (const void *)fwd_row_kernel<NORM, IN, MODE, 4, 1, 8, 0>;
      return nullptr;
    default: return nullptr;
  }
#undef NF8_ROW
}

template <int NORM, class IN>
static const void *pick_mode(int mode, int cfg) {
  switch (mode) {
    case MODE_PLAIN: return pick_cfg<NORM, IN, MODE_PLAIN>(cfg);
    case MODE_DELAYED: return pick_cfg<NORM, IN, MODE_DELAYED>(cfg);
    case MODE_MX: return pick_cfg<NORM, IN, MODE_MX>(cfg);
    case MODE_STATS: return pick_cfg<NORM, IN, MODE_STATS>(cfg);
    default: return nullptr;
  }
}

template <int NORM>
static const void *pick_in(int in_dtype, int mode, int cfg) {
  switch (in_dtype) {
    case DT_F32: return pick_mode<NORM, F32>(mode, cfg);
    case DT_BF16: return pick_mode<NORM, BF16>(mode, cfg);
    case DT_F16: return pick_mode<NORM, F16>(mode, cfg);
    default: return nullptr;
  }
}

const void *fwd_row_kernel_ptr(int norm, int in_dtype, int mode, int cfg) {
  return norm == NT_LAYERNORM ? pick_in<NT_LAYERNORM>(in_dtype, mode, cfg)
                              : pick_in<NT_RMSNORM>(in_dtype, mode, cfg);
}

}  // namespace nf8
