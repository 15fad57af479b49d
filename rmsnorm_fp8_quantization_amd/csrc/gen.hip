// gen.hip -- the general kernels: any hidden size and element-aligned pointers.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization";
// [NVRTC-PR] = "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request).
// [NVRTC-PR] Description and review thread: besides the tuned kernels for known row lengths
// there is a general kernel for arbitrary ones, slower but complete. These are this library's:
// the same operations as the row / tile / backward kernels ([XLA-Norm] Description, I/O
// Contract), on single elements instead of 16-byte strips, so the row length and the
// alignment of the tensors are free.
//
// Forward rows: one wave per row; lane l handles the elements l, l + 64, l + 128, ... (every
// load and store instruction covers 64 consecutive elements). The row is read three times
// (mean, squared deviations, output), the later passes from the caches. An MXFP8 block of 32
// elements is one half-wave.
// Forward columnwise output: a wave owns 64 consecutive columns and a block of 32 rows, taking
// the row statistics written by the row pass.
// Backward: one wave per row for dx (two passes over the row); the weight gradients come from
// a column pass (a wave owns 64 columns and a chunk of rows) whose partials the finalize
// kernel adds.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nf8 {

namespace {

template <class T> __device__ __forceinline__ float ld1(const void *base, int64_t i);
template <> __device__ __forceinline__ float ld1<F32>(const void *base, int64_t i) {
  return static_cast<const float *>(base)[i];
}
template <> __device__ __forceinline__ float ld1<BF16>(const void *base, int64_t i) {
  return __uint_as_float((uint32_t)static_cast<const uint16_t *>(base)[i] << 16);
}
template <> __device__ __forceinline__ float ld1<F16>(const void *base, int64_t i) {
  return (float)__builtin_bit_cast(_Float16, static_cast<const uint16_t *>(base)[i]);
}

// one weight of runtime dtype
__device__ __forceinline__ float ldw(const void *base, int64_t i, int dt) {
  if (dt == DT_F32) return static_cast<const float *>(base)[i];
  const uint16_t h = static_cast<const uint16_t *>(base)[i];
  return dt == DT_BF16 ? __uint_as_float((uint32_t)h << 16) : (float)__builtin_bit_cast(_Float16, h);
}

// one value stored in a runtime dtype (F32 / F16 / BF16), nearest-even
__device__ __forceinline__ void st1(void *base, int64_t i, float v, int dt) {
  if (dt == DT_F32) {
    static_cast<float *>(base)[i] = v;
  } else if (dt == DT_BF16) {
    const __bf16 h = (__bf16)v;
    static_cast<uint16_t *>(base)[i] = __builtin_bit_cast(uint16_t, h);
  } else {
    const _Float16 h = (_Float16)v;
    static_cast<uint16_t *>(base)[i] = __builtin_bit_cast(uint16_t, h);
  }
}

// one FP8 code: clamped to the largest finite value, then nearest-even
__device__ __forceinline__ uint8_t fp8_code1(float u, int fmt) {
  const float m = fp8_max(fmt);
  const float c = __builtin_amdgcn_fmed3f(u, -m, m);
  const int w = fmt == DT_E4M3 ? __builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false)
                               : __builtin_amdgcn_cvt_pk_bf8_f32(c, 0.0f, 0, false);
  return (uint8_t)(w & 0xff);
}

// Compensated (Neumaier) running sum: a lane of the general kernels adds up to H / 64 terms of
// a row in sequence, and the compensation keeps the total within a few ulps however long the
// row is (a plain float32 running sum drifts by about sqrt(n) ulps).
struct CSum {
  float s = 0.0f, c = 0.0f;
  __device__ __forceinline__ void add(float v) {
    const float t = s + v;
    c += fabsf(s) >= fabsf(v) ? (s - t) + v : (v - t) + s;
    s = t;
  }
  __device__ __forceinline__ float value() const { return s + c; }
};

// max over the 32 lanes of a half-wave (lanes l and l ^ 1, ^ 2, mirrored 8 / 16, ^ 16)
__device__ __forceinline__ float halfwave_max(float v) {
  v = fmaxf(v, xor1(v));
  v = fmaxf(v, xor2(v));
  v = fmaxf(v, hmirror(v));
  v = fmaxf(v, mirror(v));
  return fmaxf(v, xor16(v));
}

}  // namespace

// ---- forward rows -------------------------------------------------------------------------
template <int NORM, class IN, int MODE>
__global__ __launch_bounds__(256) void fwd_gen_row_kernel(FwdRowParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t H = p.hidden;
  const int fmt = p.out_dtype;
  const float inv_h = 1.0f / (float)H;
  const int64_t nj = (H + 63) / 64;  // element groups of the row

  __shared__ uint32_t s_epoch, s_last;
  __shared__ float wred[4];
  uint32_t tag = 0;
  float scale = 1.0f;
  if constexpr (MODE == MODE_DELAYED) {
    scale = *p.scale;
    tag = epoch_tag(read_epoch(p.ws, &s_epoch));
  }
  float amax_local = 0.0f;

  for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < p.rows; row += (int64_t)gridDim.x * 4) {
    const void *xr = static_cast<const char *>(p.x) + row * H * IN::bytes;
    float mean = 0.0f;
    float m2;
    if constexpr (NORM == NT_LAYERNORM) {
      // deviations from a shift K near the mean (a plain first estimate of it), so that a large
      // common part of the row does not swamp them (x - K is exact for values within a factor
      // of two of K); the mean is then K + (mean - K), rounded once
      CSum s0;
      for (int64_t j = 0; j < nj; ++j) {
        const int64_t i = j * 64 + lane;
        s0.add(i < H ? ld1<IN>(xr, i) : 0.0f);
      }
      const float shift = first_lane(wave_sum(s0.value()) * inv_h);  // rounded once (no fma fusion into x - K)
      CSum s;
      for (int64_t j = 0; j < nj; ++j) {
        const int64_t i = j * 64 + lane;
        s.add(i < H ? ld1<IN>(xr, i) - shift : 0.0f);
      }
      const float ms = wave_sum(s.value()) * inv_h;
      CSum q;
      for (int64_t j = 0; j < nj; ++j) {
        const int64_t i = j * 64 + lane;
        const float d = i < H ? (ld1<IN>(xr, i) - shift) - ms : 0.0f;
        q.add(d * d);
      }
      mean = shift + ms;
      m2 = wave_sum(q.value());
    } else {
      CSum q;
      for (int64_t j = 0; j < nj; ++j) {
        const int64_t i = j * 64 + lane;
        const float v = i < H ? ld1<IN>(xr, i) : 0.0f;
        q.add(v * v);
      }
      m2 = wave_sum(q.value());
    }
    const float rs = __builtin_amdgcn_rsqf(m2 * inv_h + p.eps);
    if (lane == 0) {
      if (p.rsigma) p.rsigma[row] = rs;
      if constexpr (NORM == NT_LAYERNORM) {
        if (p.mu) p.mu[row] = mean;
      }
    }
    if constexpr (MODE == MODE_STATS) continue;

    for (int64_t j = 0; j < nj; ++j) {
      const int64_t i = j * 64 + lane;
      const bool ok = i < H;
      float y = 0.0f;
      if (ok) {
        const float xv = ld1<IN>(xr, i);
        float g = ldw(p.gamma, i, p.w_dtype);
        if (p.zero_centered) g += 1.0f;
        if constexpr (NORM == NT_LAYERNORM) y = fmaf((xv - mean) * rs, g, ldw(p.beta, i, p.w_dtype));
        else y = (xv * rs) * g;
      }
      if constexpr (MODE == MODE_PLAIN) {
        if (ok) st1(p.y, row * H + i, y, fmt);
      } else if constexpr (MODE == MODE_DELAYED) {
        if (ok) {
          amax_local = fmaxf(amax_local, fabsf(y));
          if (p.y) static_cast<uint8_t *>(p.y)[row * H + i] = fp8_code1(y * scale, fmt);
        }
      } else {  // MODE_MX: the 32 elements of a half-wave form one block
        const float a = halfwave_max(ok ? fabsf(y) : 0.0f);
        const int X = mx_exponent(a, fmt, p.mx_ceil);
        if (ok) {
          static_cast<uint8_t *>(p.y)[row * H + i] = fp8_code1(y * exp2_neg(X), fmt);
          if ((lane & 31) == 0) static_cast<uint8_t *>(p.scale_inv)[row * p.mx_cols + (i >> 5)] = (uint8_t)(X + 127);
        }
      }
    }
  }

  if constexpr (MODE == MODE_DELAYED) {
    const float m = wave_max(amax_local);
    if (lane == 0) wred[wave] = m;
    __syncthreads();
    if (tid == 0) {
      publish_amax(p.ws, fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3])), tag);
      if (blockIdx.x == 0 && p.scale_inv) *static_cast<float *>(p.scale_inv) = 1.0f / scale;
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

// ---- forward columnwise output ------------------------------------------------------------
// item = (64-column group, 32-row block); lane = column; the row statistics come from st_mu /
// st_rs. CRM: the columnwise output in the [rows, hidden] orientation.
template <int NORM, class IN, int MODE, bool CRM>
__global__ __launch_bounds__(64) void fwd_gen_col_kernel(FwdTileParams tp) {
  const FwdRowParams &p = tp.f;
  const int lane = threadIdx.x;
  const int64_t H = p.hidden;
  const int64_t N = p.rows;
  const int fmt = p.out_dtype;
  const int64_t groups = (H + 63) / 64;
  const int64_t items = groups * tp.mx_rows;
  float scale = 1.0f;
  if constexpr (MODE == MODE_DELAYED) {
    scale = *p.scale;
    if (blockIdx.x == 0 && lane == 0 && tp.col_scale_inv) *static_cast<float *>(tp.col_scale_inv) = 1.0f / scale;
  }
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t rb = it / groups;
    const int64_t c = (it - rb * groups) * 64 + lane;
    const bool cv = c < H;
    const int64_t r0 = rb * 32;
    const int nr = (int)(N - r0 < 32 ? N - r0 : 32);
    float g = 0.0f, bt = 0.0f;
    if (cv) {
      g = ldw(p.gamma, c, p.w_dtype);
      if (p.zero_centered) g += 1.0f;
      if constexpr (NORM == NT_LAYERNORM) bt = ldw(p.beta, c, p.w_dtype);
    }
    float y[32];
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      y[k] = 0.0f;
      if (cv && k < nr) {
        const int64_t r = r0 + k;
        const float xv = ld1<IN>(p.x, r * H + c);
        if constexpr (NORM == NT_LAYERNORM) y[k] = fmaf((xv - tp.st_mu[r]) * tp.st_rs[r], g, bt);
        else y[k] = (xv * tp.st_rs[r]) * g;
        a = fmaxf(a, fabsf(y[k]));
      }
    }
    float f = scale;
    if constexpr (MODE == MODE_MX) {
      const int X = mx_exponent(a, fmt, p.mx_ceil);
      f = exp2_neg(X);
      if (cv) {
        uint8_t *sc = static_cast<uint8_t *>(tp.col_scale_inv);
        if constexpr (CRM) sc[rb * tp.mx_col_ld + c] = (uint8_t)(X + 127);
        else sc[c * tp.mx_col_ld + rb] = (uint8_t)(X + 127);
      }
    }
    if (cv) {
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        if (k < nr) {
          const uint8_t code = fp8_code1(y[k] * f, fmt);
          if constexpr (CRM) static_cast<uint8_t *>(tp.y_col)[(r0 + k) * H + c] = code;
          else static_cast<uint8_t *>(tp.y_col)[c * N + r0 + k] = code;
        }
      }
    }
  }
}

// ---- backward -----------------------------------------------------------------------------
// dx, one wave per row
template <int NORM, class IN, bool ADD>
__global__ __launch_bounds__(256) void bwd_gen_row_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t H = p.hidden;
  const float inv_h = 1.0f / (float)H;
  const int64_t nj = (H + 63) / 64;
  for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < p.rows; row += (int64_t)gridDim.x * 4) {
    const int64_t o = row * H;
    const float rs = p.rsigma[row];
    const float mu = NORM == NT_LAYERNORM ? p.mu[row] : 0.0f;
    float s1 = 0.0f, s2 = 0.0f;
    for (int64_t j = 0; j < nj; ++j) {
      const int64_t i = j * 64 + lane;
      if (i < H) {
        float g = ldw(p.gamma, i, p.w_dtype);
        if (p.zero_centered) g += 1.0f;
        const float w = ld1<IN>(p.dy, o + i) * g;
        const float xh = (ld1<IN>(p.x, o + i) - mu) * rs;
        s1 += w;
        s2 = fmaf(w, xh, s2);
      }
    }
    if constexpr (NORM == NT_LAYERNORM) s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    const float c1 = NORM == NT_LAYERNORM ? s1 * inv_h : 0.0f;
    const float c2 = s2 * inv_h;
    for (int64_t j = 0; j < nj; ++j) {
      const int64_t i = j * 64 + lane;
      if (i < H) {
        float g = ldw(p.gamma, i, p.w_dtype);
        if (p.zero_centered) g += 1.0f;
        const float w = ld1<IN>(p.dy, o + i) * g;
        const float xh = (ld1<IN>(p.x, o + i) - mu) * rs;
        float d = rs * (w - fmaf(xh, c2, c1));
        if constexpr (ADD) d += ld1<IN>(p.residual, o + i);
        st1(p.dx, o + i, d, IN::code);
      }
    }
  }
}

// weight-gradient partials: item = (64-column group, row chunk ch of p.rows / G rows); the
// partial of chunk ch goes where the backward kernel's workgroup ch would put it
template <int NORM, class IN>
__global__ __launch_bounds__(64) void bwd_gen_wgrad_kernel(BwdParams p) {
  const int lane = threadIdx.x;
  const int64_t H = p.hidden;
  const int64_t groups = (H + 63) / 64;
  const int64_t items = groups * p.G;
  const int64_t chunk = (p.rows + p.G - 1) / p.G;
  const int64_t arr = (int64_t)p.G * ((H + 31) & ~(int64_t)31);
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t ch = it / groups;
    const int64_t c = (it - ch * groups) * 64 + lane;
    if (c >= H) continue;
    float dg = 0.0f, db = 0.0f;
    const int64_t r1 = (ch + 1) * chunk < p.rows ? (ch + 1) * chunk : p.rows;
    for (int64_t r = ch * chunk; r < r1; ++r) {
      const float dy = ld1<IN>(p.dy, r * H + c);
      const float mu = NORM == NT_LAYERNORM ? p.mu[r] : 0.0f;
      const float xh = (ld1<IN>(p.x, r * H + c) - mu) * p.rsigma[r];
      dg = fmaf(dy, xh, dg);
      if constexpr (NORM == NT_LAYERNORM) db += dy;
    }
    const int64_t at = ((c >> 5) * p.G + ch) * 32 + (c & 31);
    p.part[at] = dg;
    if constexpr (NORM == NT_LAYERNORM) p.part[arr + at] = db;
  }
}

// ---- pickers --------------------------------------------------------------------------------
template <int NORM, class IN>
static const void *gen_row_mode(int mode) {
  switch (mode) {
    case MODE_PLAIN: return (const void *)fwd_gen_row_kernel<NORM, IN, MODE_PLAIN>;
    case MODE_DELAYED: return (const void *)fwd_gen_row_kernel<NORM, IN, MODE_DELAYED>;
    case MODE_MX: return (const void *)fwd_gen_row_kernel<NORM, IN, MODE_MX>;
    case MODE_STATS: return (const void *)fwd_gen_row_kernel<NORM, IN, MODE_STATS>;
    default: return nullptr;
  }
}
template <int NORM, class IN>
static const void *gen_col_mode(int mode, bool crm) {
  switch (mode) {
    case MODE_DELAYED:
      return crm ? (const void *)fwd_gen_col_kernel<NORM, IN, MODE_DELAYED, true>
                 : (const void *)fwd_gen_col_kernel<NORM, IN, MODE_DELAYED, false>;
    case MODE_MX:
      return crm ? (const void *)fwd_gen_col_kernel<NORM, IN, MODE_MX, true>
                 : (const void *)fwd_gen_col_kernel<NORM, IN, MODE_MX, false>;
    default: return nullptr;
  }
}

#define NF8_BY_IN(FN, ...)                                              \
  switch (in_dtype) {                                                   \
    case DT_F32: return FN<NORM, F32>(__VA_ARGS__);                     \
    case DT_BF16: return FN<NORM, BF16>(__VA_ARGS__);                   \
    case DT_F16: return FN<NORM, F16>(__VA_ARGS__);                     \
    default: return nullptr;                                            \
  }

template <int NORM> static const void *gen_row_in(int in_dtype, int mode) { NF8_BY_IN(gen_row_mode, mode) }
template <int NORM> static const void *gen_col_in(int in_dtype, int mode, bool crm) { NF8_BY_IN(gen_col_mode, mode, crm) }

template <int NORM, class IN>
static const void *gen_bwd_add(bool add) {
  if constexpr (NORM == NT_RMSNORM)
    return add ? (const void *)bwd_gen_row_kernel<NORM, IN, true> : (const void *)bwd_gen_row_kernel<NORM, IN, false>;
  else
    return add ? nullptr : (const void *)bwd_gen_row_kernel<NORM, IN, false>;
}
template <int NORM, class IN>
static const void *gen_wgrad(int) { return (const void *)bwd_gen_wgrad_kernel<NORM, IN>; }
template <int NORM> static const void *gen_bwd_in(int in_dtype, bool add) { NF8_BY_IN(gen_bwd_add, add) }
template <int NORM> static const void *gen_wgrad_in(int in_dtype) { NF8_BY_IN(gen_wgrad, 0) }
#undef NF8_BY_IN

const void *fwd_gen_row_kernel_ptr(int norm, int in_dtype, int mode) {
  return norm == NT_LAYERNORM ? gen_row_in<NT_LAYERNORM>(in_dtype, mode) : gen_row_in<NT_RMSNORM>(in_dtype, mode);
}
const void *fwd_gen_col_kernel_ptr(int norm, int in_dtype, int mode, bool col_rowmajor) {
  return norm == NT_LAYERNORM ? gen_col_in<NT_LAYERNORM>(in_dtype, mode, col_rowmajor)
                              : gen_col_in<NT_RMSNORM>(in_dtype, mode, col_rowmajor);
}
const void *bwd_gen_row_kernel_ptr(int norm, int in_dtype, bool add) {
  return norm == NT_LAYERNORM ? gen_bwd_in<NT_LAYERNORM>(in_dtype, add) : gen_bwd_in<NT_RMSNORM>(in_dtype, add);
}
const void *bwd_gen_wgrad_kernel_ptr(int norm, int in_dtype) {
  return norm == NT_LAYERNORM ? gen_wgrad_in<NT_LAYERNORM>(in_dtype) : gen_wgrad_in<NT_RMSNORM>(in_dtype);
}

}  // namespace nf8
