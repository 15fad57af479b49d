// fwd_row.hip -- LayerNorm / RMSNorm forward with a fused output epilogue, one row per team.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization".
// [XLA-Norm] Overview / Description: LayerNorm or RMSNorm forward that writes the normalised
// output (optionally FP8-quantised with delayed per-tensor or MXFP8 block scaling, in the
// same kernel launch) plus mu (LayerNorm) and rsigma for the backward. [XLA-Norm] I/O Contract
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

template <int NORM, class IN, int MODE, int P, int T, int KC>
__global__ __launch_bounds__(64 * P * T) void fwd_row_kernel(FwdRowParams p) {
  constexpr int TEAM = 64 * P;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int team = wave / P;
  const int wt = wave - team * P;
  const int tl = tid - team * TEAM;
  const int64_t H = p.hidden;
  const int fmt = p.out_dtype;

  // columns of this lane, effective weight (1 + gamma when zero-centred) and beta
  bool cv[KC];
  float g[KC][8];
  float b[NORM == NT_LAYERNORM ? KC : 1][8];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int64_t col = 8 * (int64_t)(tl + TEAM * k);
    cv[k] = col < H;
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
  float scale = 1.0f;
  if constexpr (MODE == MODE_DELAYED) scale = *p.scale;
  float amax_local = 0.0f;

  __shared__ Stats red[2][T][P];
  const float inv_h = 1.0f / (float)H;

  int iter = 0;
  for (int64_t base = (int64_t)blockIdx.x * T; base < p.rows; base += (int64_t)gridDim.x * T, ++iter) {
    const int64_t row = base + team;
    const bool rv = row < p.rows;
    Strip<IN> xs[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      if (rv && cv[k]) load_strip<IN>(xs[k], p.x, row * H + 8 * (int64_t)(tl + TEAM * k));
      else zero_strip<IN>(xs[k]);
    }

    // ---- lane-local statistics over its valid strips
    Stats st{0.0f, 0.0f, 0.0f};
    if constexpr (NORM == NT_LAYERNORM) {
      float s = 0.0f, n = 0.0f;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xv[8];
        strip_to_f32<IN>(xs[k], xv);
        if (rv && cv[k]) {
#pragma unroll
          for (int i = 0; i < 8; ++i) s += xv[i];
          n += 8.0f;
        }
      }
      const float m = n > 0.0f ? s / n : 0.0f;
      float q = 0.0f;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xv[8];
        strip_to_f32<IN>(xs[k], xv);
        if (rv && cv[k]) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float d = xv[i] - m;
            q = fmaf(d, d, q);
          }
        }
      }
      st = Stats{n, m, q};
      st = wave_merge(st);
    } else {
      float q = 0.0f;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xv[8];
        strip_to_f32<IN>(xs[k], xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) q = fmaf(xv[i], xv[i], q);  // masked strips are zero
      }
      st.m2 = wave_sum(q);
    }

    // ---- merge the team's waves in a fixed order
    if constexpr (P > 1) {
      if (lane == 0) red[iter & 1][team][wt] = st;
      __syncthreads();
      st = red[iter & 1][team][0];
#pragma unroll
      for (int w = 1; w < P; ++w) {
        const Stats o = red[iter & 1][team][w];
        if constexpr (NORM == NT_LAYERNORM) st = chan_merge(st, o);
        else st.m2 += o.m2;
      }
    }

    float mu = 0.0f, rs;
    if constexpr (NORM == NT_LAYERNORM) {
      mu = st.mean;
      rs = 1.0f / sqrtf(st.m2 * inv_h + p.eps);
    } else {
      rs = 1.0f / sqrtf(st.m2 * inv_h + p.eps);
    }
    if (rv && tl == 0) {
      if (p.rsigma) p.rsigma[row] = rs;
      if constexpr (NORM == NT_LAYERNORM) {
        if (p.mu) p.mu[row] = mu;
      }
    }

    // ---- normalise and store
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const bool ok = rv && cv[k];
      const int64_t col = 8 * (int64_t)(tl + TEAM * k);
      float xv[8], y[8];
      strip_to_f32<IN>(xs[k], xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (NORM == NT_LAYERNORM) y[i] = fmaf((xv[i] - mu) * rs, g[k][i], b[k][i]);
        else y[i] = (xv[i] * rs) * g[k][i];
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
        if (ok) *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(p.y) + row * H + col) = c;
      } else {  // MODE_MX: 4 consecutive lanes hold one 32-element block
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(y[i]));
        a = quad_max(ok ? a : 0.0f);
        const int X = mx_exponent(a, fmt);
        const float f = exp2_neg(X);
        float u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = y[i] * f;
        const uint2 c = fp8_pack8(u, fmt);
        if (ok) {
          *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(p.y) + row * H + col) = c;
          if ((tl & 3) == 0)
            static_cast<uint8_t *>(p.scale_inv)[row * p.mx_cols + (col >> 5)] = (uint8_t)(X + 127);
        }
      }
    }
  }

  if constexpr (MODE == MODE_DELAYED) {
    // tensor amax: wave max -> one atomic max per wave -> the last workgroup to finish
    // publishes max(amax_in, amax) and re-zeroes the header words it used
    const float m = wave_max(amax_local);
    if (lane == 0) max_dev(p.ws + kWsAmax, __float_as_uint(m));
    vmem_drain();
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = add_dev(p.ws + kWsDone, 1u);
      if (prev == gridDim.x - 1) {
        const float tot = __uint_as_float(xchg_dev(p.ws + kWsAmax, 0u));
        *p.updated_amax = fmaxf(*p.amax_in, tot);
        xchg_dev(p.ws + kWsDone, 0u);
      }
      if (blockIdx.x == 0) *static_cast<float *>(p.scale_inv) = 1.0f / scale;
    }
  }
}

// ------------------------------------------------------------------------------------------
// instantiation table
// ------------------------------------------------------------------------------------------

template <int NORM, class IN, int MODE>
static const void *pick_cfg(int cfg) {
  switch (cfg) {
    case ROW_W1_K1: return (const void *)fwd_row_kernel<NORM, IN, MODE, 1, 4, 1>;
    case ROW_W1_K2: return (const void *)fwd_row_kernel<NORM, IN, MODE, 1, 4, 2>;
    case ROW_W1_K4: return (const void *)fwd_row_kernel<NORM, IN, MODE, 1, 4, 4>;
    case ROW_W1_K8: return (const void *)fwd_row_kernel<NORM, IN, MODE, 1, 4, 8>;
    case ROW_W4_K2: return (const void *)fwd_row_kernel<NORM, IN, MODE, 4, 1, 2>;
    case ROW_W4_K4: return (const void *)fwd_row_kernel<NORM, IN, MODE, 4, 1, 4>;
    case ROW_W8_K4: return (const void *)fwd_row_kernel<NORM, IN, MODE, 8, 1, 4>;
    case ROW_W2T2_K4: return (const void *)fwd_row_kernel<NORM, IN, MODE, 2, 2, 4>;
    case ROW_W8_K1: return (const void *)fwd_row_kernel<NORM, IN, MODE, 8, 1, 1>;
    case ROW_W4T2_K2: return (const void *)fwd_row_kernel<NORM, IN, MODE, 4, 2, 2>;
    default: return nullptr;
  }
}

template <int NORM, class IN>
static const void *pick_mode(int mode, int cfg) {
  switch (mode) {
    case MODE_PLAIN: return pick_cfg<NORM, IN, MODE_PLAIN>(cfg);
    case MODE_DELAYED: return pick_cfg<NORM, IN, MODE_DELAYED>(cfg);
    case MODE_MX: return pick_cfg<NORM, IN, MODE_MX>(cfg);
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
