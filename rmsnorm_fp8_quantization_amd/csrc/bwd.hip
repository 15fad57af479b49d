// bwd.hip -- LayerNorm / RMSNorm backward (optionally fused with the residual-gradient add)
// and the weight-gradient finalize kernel.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization";
// [BwdAdd]   = "Implementation: NVIDIA TransformerEngine Ops Fused Backward Add RMSNorm";
// [NVRTC-PR] = "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request).
// [XLA-Norm] Description: the backward dispatch for both norm types. [NVRTC-PR] file table
// and Flowchart: the backward kernels leave per-CTA weight-gradient partials ("semi" kernels)
// and a finalize kernel reduces them. [BwdAdd] Overview / Description / I/O Contract: the
// RMSNorm backward adds the residual branch's gradient into dx inside the same kernel, and
// returns the weight gradient.
//
// Work split: all W waves of a workgroup work on one row at a time; lane t owns the strips
// t + 64 * W * k. The grid is persistent (G workgroups, rows g, g + G, ...), so each lane keeps
// its columns' gamma and its dgamma / dbeta partial sums in registers across rows and writes
// them once; the finalize kernel adds the G partial rows in a fixed order (deterministic).
#include "device_common.hpp"
#include "kernels.hpp"

namespace nf8 {

template <int NORM, class IN, bool ADD, int W, int KC, int T>
__global__ __launch_bounds__(64 * W * T) void bwd_kernel(BwdParams p) {
  constexpr int NT = 64 * W;  // threads of one team (one row)
  const int lane = threadIdx.x & 63;
  // (the team is the same for every lane of a wave: taken through readfirstlane so that row
  // indices and row addresses are scalar)
  const int team = __builtin_amdgcn_readfirstlane((int)threadIdx.x / NT);
  const int tid = (int)threadIdx.x - team * NT;  // thread within the team
  const int wave = tid >> 6;                      // wave within the team
  const int64_t H = p.hidden;

  bool cv[KC];
  float g[KC][8], dg[KC][8], db[NORM == NT_LAYERNORM ? KC : 1][8];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int64_t col = 8 * (int64_t)(tid + NT * k);
    cv[k] = col < H;
    if (cv[k]) {
      load_w8(g[k], p.gamma, col, p.w_dtype);
      if (p.zero_centered) {
#pragma unroll
        for (int i = 0; i < 8; ++i) g[k][i] += 1.0f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) g[k][i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dg[k][i] = 0.0f;
      if constexpr (NORM == NT_LAYERNORM) db[k][i] = 0.0f;
    }
  }

  __shared__ float red[2][T][W][2];
  const float inv_h = 1.0f / (float)H;

  // The next row's dy, x (and residual) are loaded while the current row is processed. Every
  // load and store is issued on every path (buffer accesses whose offset is moved past the
  // row's end where a lane has nothing to read or write): under a branch an access may not
  // have been issued, and the wait before the next use of an earlier load would then drain
  // every access in flight, the next row's loads included.
  struct RowData {
    Strip<IN> dys[KC], xs[KC], rsd[ADD ? KC : 1];
    float rs, mu;
  };
  // (a strip past the end of the row, or of a row past the last, reads zeros)
  const uint32_t row_bytes = (uint32_t)(H * IN::bytes);
  auto load_row = [&](RowData &d, int64_t base) {
    const int64_t row = base + team;
    const bool in = row < p.rows;
    const int64_t r = in ? row : 0;
    const nf8_rsrc rdy = make_rsrc(static_cast<const char *>(p.dy) + r * row_bytes, row_bytes);
    const nf8_rsrc rx = make_rsrc(static_cast<const char *>(p.x) + r * row_bytes, row_bytes);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const uint32_t off = in && cv[k] ? (uint32_t)(8 * IN::bytes * (tid + NT * k)) : kOffNone;
      load_strip_at<IN>(d.dys[k], rdy, off);
      load_strip_at<IN>(d.xs[k], rx, off);
      if constexpr (ADD)
        load_strip_at<IN>(d.rsd[k], make_rsrc(static_cast<const char *>(p.residual) + r * row_bytes, row_bytes), off);
    }
    d.rs = p.rsigma[r];
    d.mu = NORM == NT_LAYERNORM ? p.mu[r] : 0.0f;
  };

  // one row: statistics, dx, and the weight-gradient partial sums
  auto step = [&](RowData &cur, int64_t base, int iter) {
    const int64_t row = base + team;
    const bool rv = row < p.rows;  // a team past the last row adds nothing and stores nothing
    const Strip<IN> *const dys = cur.dys;
    const Strip<IN> *const xs = cur.xs;
    const Strip<IN> *const rsd = cur.rsd;
    const float rs = cur.rs;
    const float mu = cur.mu;

    // row sums of w = dy * g and w * xhat
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float dv[8], xv[8];
      strip_to_f32<IN>(dys[k], dv);
      strip_to_f32<IN>(xs[k], xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xh = (xv[i] - mu) * rs;
        const float w = dv[i] * g[k][i];
        s1 += w;
        s2 = fmaf(w, xh, s2);
      }
    }
    if constexpr (NORM == NT_LAYERNORM) s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    if constexpr (W > 1) {
      if (lane == 0) {
        red[iter & 1][team][wave][0] = s1;
        red[iter & 1][team][wave][1] = s2;
      }
      __syncthreads();
      s1 = red[iter & 1][team][0][0];
      s2 = red[iter & 1][team][0][1];
#pragma unroll
      for (int w = 1; w < W; ++w) {
        s1 += red[iter & 1][team][w][0];
        s2 += red[iter & 1][team][w][1];
      }
    }
    // dx of this row through a resource that covers the row (the team's row is the same for
    // every lane of a wave)
    const nf8_rsrc rdx = make_rsrc(static_cast<char *>(p.dx) + (rv ? row : 0) * row_bytes, row_bytes);
    const float c1 = NORM == NT_LAYERNORM ? s1 * inv_h : 0.0f;
    const float c2 = s2 * inv_h;

#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float dv[8], xv[8], out[8];
      strip_to_f32<IN>(dys[k], dv);
      strip_to_f32<IN>(xs[k], xv);
      float res[8];
      if constexpr (ADD) strip_to_f32<IN>(rsd[k], res);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xh = (xv[i] - mu) * rs;
        const float w = dv[i] * g[k][i];
        float d = rs * (w - fmaf(xh, c2, c1));
        if constexpr (ADD) d += res[i];
        out[i] = d;
        dg[k][i] = fmaf(dv[i], xh, dg[k][i]);
        if constexpr (NORM == NT_LAYERNORM) db[k][i] += dv[i];
      }
      store_t8_at<IN>(rdx, rv && cv[k] ? (uint32_t)(8 * IN::bytes * (tid + NT * k)) : kOffNone, out);
    }
  };

  // Two row buffers used in turn, so that the next row's loads never wait on the current
  // row's registers. (Not for 16 waves x 2 strips, nor for float32 rows of 3 strips per lane:
  // two rows of inputs would not fit the register budget; those load each row after the
  // previous one is done.)
  constexpr bool PF = !(W == 16 && KC >= 2) && !(IN::bytes == 4 && KC >= 3);
  // (T teams walk rows base + team in step, so every team makes the same number of steps and
  // meets every barrier)
  // The workgroup's n steps (base rows first, first + G, ...) run as n / 2 two-step trips and
  // a last single step: a loop with one exit (a break between the two steps would join the
  // back edge on a path where the next row's loads are never used, and every trip would then
  // wait for all accesses in flight before issuing its loads).
  const int64_t G = (int64_t)gridDim.x * T;
  const int64_t first = (int64_t)blockIdx.x * T;
  const int64_t n = first < p.rows ? (p.rows - first + G - 1) / G : 0;
  RowData a, b;
  load_row(a, first);
  int64_t row = first;
  int iter = 0;
  if constexpr (PF) {
    for (int64_t q = n >> 1; q > 0; --q) {
      // (the scheduling barriers keep each row's work below the next row's loads: work on a
      // row moved above them would make the loads wait for that row's own loads)
      load_row(b, row + G);
      __builtin_amdgcn_sched_barrier(0);
      step(a, row, iter);
      load_row(a, row + 2 * G);
      __builtin_amdgcn_sched_barrier(0);
      step(b, row + G, iter + 1);
      row += 2 * G;
      iter += 2;
    }
    if (n & 1) step(a, row, iter);
  } else {
    // one buffer: each row's loads go out after the previous row is done
    for (int64_t q = n; q > 0; --q) {
      step(a, row, iter);
      load_row(a, row + G);
      row += G;
      ++iter;
    }
  }

  // the teams' weight-gradient sums, added in team order (deterministic)
  if constexpr (T > 1) {
    constexpr int NW = NORM == NT_LAYERNORM ? 2 : 1;
    __shared__ __align__(16) float tpart[T > 1 ? (T - 1) * NW * KC * 8 * NT : 1];
    if (team > 0) {
      float *d = tpart + (size_t)(team - 1) * NW * KC * 8 * NT;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          d[(k * 8 + i) * NT + tid] = dg[k][i];
          if constexpr (NORM == NT_LAYERNORM) d[((KC + k) * 8 + i) * NT + tid] = db[k][i];
        }
      }
    }
    __syncthreads();
    if (team > 0) return;
#pragma unroll
    for (int t = 1; t < T; ++t) {
      const float *d = tpart + (size_t)(t - 1) * NW * KC * 8 * NT;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dg[k][i] += d[(k * 8 + i) * NT + tid];
          if constexpr (NORM == NT_LAYERNORM) db[k][i] += d[((KC + k) * 8 + i) * NT + tid];
        }
      }
    }
  }

  // this workgroup's partial weight gradients, into the column-block-major layout
  // [H32 / 32][G][32] (H32 = hidden rounded up to 32): each 32-column block's G partials are
  // contiguous, so the finalize kernel streams them
  const int64_t arr = (int64_t)p.G * ((H + 31) & ~(int64_t)31);
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    if (!cv[k]) continue;
    const int64_t col = 8 * (int64_t)(tid + NT * k);
    const int64_t at = ((col >> 5) * p.G + blockIdx.x) * 32 + (col & 31);
    float4 *dst = reinterpret_cast<float4 *>(p.part + at);
    dst[0] = make_float4(dg[k][0], dg[k][1], dg[k][2], dg[k][3]);
    dst[1] = make_float4(dg[k][4], dg[k][5], dg[k][6], dg[k][7]);
    if constexpr (NORM == NT_LAYERNORM) {
      float4 *dsb = reinterpret_cast<float4 *>(p.part + arr + at);
      dsb[0] = make_float4(db[k][0], db[k][1], db[k][2], db[k][3]);
      dsb[1] = make_float4(db[k][4], db[k][5], db[k][6], db[k][7]);
    }
  }
}

// Fixed-order reduction of the G partials. Workgroup (x, y) owns column block x (32 columns)
// of array y (0: dgamma, 1: dbeta), whose G partials are one contiguous [G][32] slab; thread
// (c, q) adds 4 columns (one float4) of partials q, q + 32, q + 64, ... with eight loads in
// flight (each load instruction reads 4 KB of the slab), and the 32 sums per column are added
// in a fixed order (groups of four q, then the eight groups). The grid has ceil(H / 32)
// workgroups per array.
__global__ __launch_bounds__(256) void bwd_finalize_kernel(FinalizeParams p) {
  constexpr int Q = 32;
  const int c = threadIdx.x & 7;
  const int q = threadIdx.x >> 3;
  const int64_t col = (int64_t)blockIdx.x * 32 + 4 * c;
  const int which = blockIdx.y;
  const int64_t arr = (int64_t)p.G * ((p.hidden + 31) & ~(int64_t)31);
  const float *part = p.part + which * arr + (int64_t)blockIdx.x * p.G * 32 + 4 * c;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (col < p.hidden) {
    // eight loads in flight per thread (one round trip for G <= 256), added in g order
    int g = q;
    for (; g + 7 * Q < p.G; g += 8 * Q) {
      float4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const float4 *>(part + (int64_t)(g + j * Q) * 32);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
      }
    }
    for (; g < p.G; g += Q) {
      const float4 a = *reinterpret_cast<const float4 *>(part + (int64_t)g * 32);
      s.x += a.x; s.y += a.y; s.z += a.z; s.w += a.w;
    }
  }
  // the 32 sums of each column, in a fixed tree: eight groups of four q, then the groups
  __shared__ __align__(16) float red[Q][32];
  __shared__ float red2[8][32];
  *reinterpret_cast<float4 *>(&red[q][4 * c]) = s;
  __syncthreads();
  {
    const int j = threadIdx.x & 31, h = threadIdx.x >> 5;
    red2[h][j] = ((red[4 * h][j] + red[4 * h + 1][j]) + red[4 * h + 2][j]) + red[4 * h + 3][j];
  }
  __syncthreads();
  if (threadIdx.x < 32) {
    const int64_t out = (int64_t)blockIdx.x * 32 + threadIdx.x;
    if (out < p.hidden) {
      float t = red2[0][threadIdx.x];
#pragma unroll
      for (int h = 1; h < 8; ++h) t += red2[h][threadIdx.x];
      void *dst = which == 0 ? p.dgamma : p.dbeta;
      if (p.w_dtype == DT_F32) {
        static_cast<float *>(dst)[out] = t;
      } else if (p.w_dtype == DT_BF16) {
        __bf16 h = (__bf16)t;
        static_cast<uint16_t *>(dst)[out] = __builtin_bit_cast(uint16_t, h);
      } else {
        _Float16 h = (_Float16)t;
        static_cast<uint16_t *>(dst)[out] = __builtin_bit_cast(uint16_t, h);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------

template <int NORM, class IN, bool ADD>
static const void *pick_bwd_cfg(int cfg) {
#define NF8_BWD(C) \
  (const void *)bwd_kernel<NORM, IN, ADD, kBwdShapes[C].W, kBwdShapes[C].KC, kBwdShapes[C].T>
  switch (cfg) {
    case BWD_W2_K1: return NF8_BWD(BWD_W2_K1);
    case BWD_W4_K1: return NF8_BWD(BWD_W4_K1);
    case BWD_W4_K2: return NF8_BWD(BWD_W4_K2);
    case BWD_W8_K2: return NF8_BWD(BWD_W8_K2);
    case BWD_W16_K2: return NF8_BWD(BWD_W16_K2);
    case BWD_W8_K1: return NF8_BWD(BWD_W8_K1);
    case BWD_W16_K1: return NF8_BWD(BWD_W16_K1);
    case BWD_W4_K4: return NF8_BWD(BWD_W4_K4);
    case BWD_W2_K1_T1: return NF8_BWD(BWD_W2_K1_T1);
    case BWD_W4_K1_T1: return NF8_BWD(BWD_W4_K1_T1);
    case BWD_W4_K2_T1: return NF8_BWD(BWD_W4_K2_T1);
    case BWD_W8_K3: return NF8_BWD(BWD_W8_K3);
    case BWD_W5_K2_T2: return NF8_BWD(BWD_W5_K2_T2);
    case BWD_W5_K2_T1: return NF8_BWD(BWD_W5_K2_T1);
    default: return nullptr;
  }
#undef NF8_BWD
}

template <int NORM, bool ADD>
static const void *pick_bwd_in(int in_dtype, int cfg) {
  switch (in_dtype) {
    case DT_F32: return pick_bwd_cfg<NORM, F32, ADD>(cfg);
    case DT_BF16: return pick_bwd_cfg<NORM, BF16, ADD>(cfg);
    case DT_F16: return pick_bwd_cfg<NORM, F16, ADD>(cfg);
    default: return nullptr;
  }
}

const void *bwd_kernel_ptr(int norm, int in_dtype, bool add, int cfg) {
  if (norm == NT_LAYERNORM) return add ? nullptr : pick_bwd_in<NT_LAYERNORM, false>(in_dtype, cfg);
  return add ? pick_bwd_in<NT_RMSNORM, true>(in_dtype, cfg) : pick_bwd_in<NT_RMSNORM, false>(in_dtype, cfg);
}

const void *bwd_finalize_kernel_ptr() { return (const void *)bwd_finalize_kernel; }

// zero the workspace header
__global__ __launch_bounds__(256) void ws_init_kernel(uint32_t *ws) {
  for (int i = threadIdx.x; i < kWsHeaderBytes / 4; i += 256) ws[i] = 0u;
}
const void *ws_init_kernel_ptr() { return (const void *)ws_init_kernel; }

}  // namespace nf8
