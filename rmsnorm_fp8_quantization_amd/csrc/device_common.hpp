// device_common.hpp -- element conversions, strip loads/stores, cross-lane reductions and
// cross-workgroup synchronisation shared by the gfx950 normalisation kernels.
//
// Pages cited (by title and section):
//   [XLA-Norm]  "Implementation: NVIDIA TransformerEngine JAX XLA Normalization"
//   [BwdAdd]    "Implementation: NVIDIA TransformerEngine Ops Fused Backward Add RMSNorm"
//   [NVRTC-PR]  "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request)
//
// Data layout used by every kernel: a "strip" is 8 consecutive elements of one row, i.e. one
// 16-byte vector for 16-bit inputs (two for float32). A lane owns whole strips; consecutive
// lanes own consecutive strips so a wave's loads and stores are contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace nf8 {

// ------------------------------------------------------------------------------------------
// element types
// ------------------------------------------------------------------------------------------

struct F32 {
  static constexpr int code = DT_F32;
  static constexpr int bytes = 4;
};
struct F16 {
  static constexpr int code = DT_F16;
  static constexpr int bytes = 2;
};
struct BF16 {
  static constexpr int code = DT_BF16;
  static constexpr int bytes = 2;
};

// Raw storage of one strip: 16 bytes for 16-bit types, 32 bytes for float32.
template <class T> struct Strip;
template <> struct Strip<F32> { uint4 v[2]; };
template <> struct Strip<F16> { uint4 v[1]; };
template <> struct Strip<BF16> { uint4 v[1]; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <class T> __device__ __forceinline__ void strip_to_f32(const Strip<T> &s, float (&o)[8]);
template <> __device__ __forceinline__ void strip_to_f32<F32>(const Strip<F32> &s, float (&o)[8]) {
  o[0] = __uint_as_float(s.v[0].x); o[1] = __uint_as_float(s.v[0].y);
  o[2] = __uint_as_float(s.v[0].z); o[3] = __uint_as_float(s.v[0].w);
  o[4] = __uint_as_float(s.v[1].x); o[5] = __uint_as_float(s.v[1].y);
  o[6] = __uint_as_float(s.v[1].z); o[7] = __uint_as_float(s.v[1].w);
}
template <> __device__ __forceinline__ void strip_to_f32<BF16>(const Strip<BF16> &s, float (&o)[8]) {
  o[0] = bf16_lo(s.v[0].x); o[1] = bf16_hi(s.v[0].x);
  o[2] = bf16_lo(s.v[0].y); o[3] = bf16_hi(s.v[0].y);
  o[4] = bf16_lo(s.v[0].z); o[5] = bf16_hi(s.v[0].z);
  o[6] = bf16_lo(s.v[0].w); o[7] = bf16_hi(s.v[0].w);
}
template <> __device__ __forceinline__ void strip_to_f32<F16>(const Strip<F16> &s, float (&o)[8]) {
  o[0] = f16_lo(s.v[0].x); o[1] = f16_hi(s.v[0].x);
  o[2] = f16_lo(s.v[0].y); o[3] = f16_hi(s.v[0].y);
  o[4] = f16_lo(s.v[0].z); o[5] = f16_hi(s.v[0].z);
  o[6] = f16_lo(s.v[0].w); o[7] = f16_hi(s.v[0].w);
}

// Sum and sum of squares of a strip's 8 values. 16-bit inputs: one packed dot product per pair
// of values (with (1, 1), or with the pair itself), accumulated in binary32 -- the products of
// 16-bit values are exact in binary32 -- so a strip costs 4 instructions and no conversions.
typedef __bf16 nf8_bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 nf8_f16x2 __attribute__((ext_vector_type(2)));
template <class T> __device__ __forceinline__ float strip_sum(const Strip<T> &s);
template <> __device__ __forceinline__ float strip_sum<F32>(const Strip<F32> &s) {
  float o[8];
  strip_to_f32<F32>(s, o);
  return ((o[0] + o[1]) + (o[2] + o[3])) + ((o[4] + o[5]) + (o[6] + o[7]));
}
template <> __device__ __forceinline__ float strip_sum<BF16>(const Strip<BF16> &s) {
  const uint32_t w[4] = {s.v[0].x, s.v[0].y, s.v[0].z, s.v[0].w};
  const nf8_bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float a = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(nf8_bf16x2, w[d]), one, a, false);
  return a;
}
template <> __device__ __forceinline__ float strip_sum<F16>(const Strip<F16> &s) {
  const uint32_t w[4] = {s.v[0].x, s.v[0].y, s.v[0].z, s.v[0].w};
  const nf8_f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  float a = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) a = __builtin_amdgcn_fdot2(__builtin_bit_cast(nf8_f16x2, w[d]), one, a, false);
  return a;
}
template <class T> __device__ __forceinline__ float strip_sumsq(const Strip<T> &s);
template <> __device__ __forceinline__ float strip_sumsq<BF16>(const Strip<BF16> &s) {
  const uint32_t w[4] = {s.v[0].x, s.v[0].y, s.v[0].z, s.v[0].w};
  float a = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(nf8_bf16x2, w[d]), __builtin_bit_cast(nf8_bf16x2, w[d]), a, false);
  return a;
}
template <> __device__ __forceinline__ float strip_sumsq<F16>(const Strip<F16> &s) {
  const uint32_t w[4] = {s.v[0].x, s.v[0].y, s.v[0].z, s.v[0].w};
  float a = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    a = __builtin_amdgcn_fdot2(__builtin_bit_cast(nf8_f16x2, w[d]), __builtin_bit_cast(nf8_f16x2, w[d]), a, false);
  return a;
}

// Register-pressure barrier: makes the compiler treat a strip's packed registers as changed,
// so values converted from them before this point are not kept alive to be reused after it
// (emits no instruction).
template <class T> __device__ __forceinline__ void opaque(Strip<T> &s) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(Strip<T>) / 16); ++i)
    asm volatile("" : "+v"(s.v[i].x), "+v"(s.v[i].y), "+v"(s.v[i].z), "+v"(s.v[i].w));
}

// Streaming accesses: every input row element is read once and every output element written
// once, so rows use non-temporal loads and stores (they do not displace reused data such as the
// weights from the caches; on MI355X they also raise the achieved HBM bandwidth of a stream).
typedef unsigned int nf8_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int nf8_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_nt16(const void *p) {
  const nf8_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nf8_u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt16(void *p, uint4 v) {
  const nf8_u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<nf8_u32x4 *>(p));
}
__device__ __forceinline__ void st_nt8(void *p, uint2 v) {
  const nf8_u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<nf8_u32x2 *>(p));
}

// one strip of a row (non-temporal)
template <class T>
__device__ __forceinline__ void load_strip(Strip<T> &s, const void *base, int64_t elem) {
  const char *p = static_cast<const char *>(base) + elem * T::bytes;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(Strip<T>) / 16); ++i) s.v[i] = ld_nt16(p + 16 * i);
}
// keep a strip (ok) or zero it, without a branch
template <class T> __device__ __forceinline__ void mask_strip(Strip<T> &s, bool ok) {
  const uint32_t m = ok ? ~0u : 0u;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(Strip<T>) / 16); ++i) {
    s.v[i].x &= m;
    s.v[i].y &= m;
    s.v[i].z &= m;
    s.v[i].w &= m;
  }
}
template <class T> __device__ __forceinline__ void zero_strip(Strip<T> &s) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(Strip<T>) / 16); ++i) s.v[i] = make_uint4(0, 0, 0, 0);
}

// 8 weights (gamma or beta) of runtime dtype -> float32
__device__ __forceinline__ void load_w8(float (&o)[8], const void *base, int64_t elem, int dt) {
  if (dt == DT_F32) {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem);
    float4 a = p[0], b = p[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  } else {
    Strip<BF16> s;  // cached: the weights are reused by every row
    s.v[0] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem);
    if (dt == DT_BF16) {
      strip_to_f32<BF16>(s, o);
    } else {
      Strip<F16> h;
      h.v[0] = s.v[0];
      strip_to_f32<F16>(h, o);
    }
  }
}
// the same in two steps, so that the loads can run ahead of their use: load_w8_raw issues two
// 16-byte loads whatever the dtype (a 16-bit weight array reads its 16 bytes twice) and keeps
// the raw bits; w8_convert turns them into floats where they are used (converting at the load
// would make the compiler wait there for every load in flight)
struct W8Raw {
  uint4 a, c;
};
__device__ __forceinline__ void load_w8_raw(W8Raw &w, const void *base, uint32_t elem, int dt) {
  const bool f32 = dt == DT_F32;
  const uint32_t off = elem * (f32 ? 4u : 2u);
  const char *b = static_cast<const char *>(base);
  w.a = *reinterpret_cast<const uint4 *>(b + off);
  w.c = *reinterpret_cast<const uint4 *>(b + (off + (f32 ? 16u : 0u)));
}
__device__ __forceinline__ void w8_convert(float (&o)[8], const W8Raw &w, int dt) {
  if (dt == DT_F32) {
    const uint32_t v[8] = {w.a.x, w.a.y, w.a.z, w.a.w, w.c.x, w.c.y, w.c.z, w.c.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = __uint_as_float(v[i]);
  } else if (dt == DT_BF16) {
    Strip<BF16> s;
    s.v[0] = w.a;
    strip_to_f32<BF16>(s, o);
  } else {
    Strip<F16> h;
    h.v[0] = w.a;
    strip_to_f32<F16>(h, o);
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 ha = (__bf16)a, hb = (__bf16)b;  // v_cvt_pk_bf16_f32: nearest-even
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// store 8 float32 values as runtime out dtype (F32 / F16 / BF16) at element offset `elem`
// ---- stores issued on every path
// A store under a divergent branch leaves a path on which it was not issued. Loads and stores
// retire in issue order on one counter, so where such paths join the compiler cannot count the
// accesses issued after an earlier load, and the next use of that load waits for every access
// in flight (the next row's loads and this row's stores included). A raw buffer store whose
// offset lies at or past the resource's size is dropped by the hardware: a masked-off lane gets
// such an offset and the store instruction itself is issued on every path.
typedef __amdgpu_buffer_rsrc_t nf8_rsrc;
constexpr uint32_t kOffNone = 0x80000000u;  // an offset past every resource this library builds
constexpr int kCpolNt = 2;                   // non-temporal
__device__ __forceinline__ nf8_rsrc make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void st16_at(nf8_rsrc r, uint32_t off, uint4 v) {
  const nf8_u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, kCpolNt);
}
// a strip read through a buffer resource at byte offset off: an offset at or past the
// resource's size reads zeros (kOffNone: a zero strip)
template <class T> __device__ __forceinline__ void load_strip_at(Strip<T> &s, nf8_rsrc r, uint32_t off) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(Strip<T>) / 16); ++i) {
    const nf8_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u * (uint32_t)i, 0, kCpolNt);
    s.v[i] = make_uint4(v.x, v.y, v.z, v.w);
  }
}
// 8 float32 values stored in the storage type T at byte offset off (kOffNone: nothing stored)
template <class T> __device__ __forceinline__ void store_t8_at(nf8_rsrc r, uint32_t off, const float (&y)[8]);

__device__ __forceinline__ void store_out8(void *base, int64_t elem, const float (&y)[8], int dt) {
  if (dt == DT_F32) {
    float *p = static_cast<float *>(base) + elem;
    st_nt16(p, make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])));
    st_nt16(p + 4, make_uint4(__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]), __float_as_uint(y[7])));
  } else if (dt == DT_BF16) {
    st_nt16(static_cast<uint16_t *>(base) + elem,
            make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                       pack_bf16x2(y[6], y[7])));
  } else {
    st_nt16(static_cast<uint16_t *>(base) + elem,
            make_uint4(pack_f16x2(y[0], y[1]), pack_f16x2(y[2], y[3]), pack_f16x2(y[4], y[5]),
                       pack_f16x2(y[6], y[7])));
  }
}

template <class T> __device__ __forceinline__ void store_t8_at(nf8_rsrc r, uint32_t off, const float (&y)[8]) {
  if constexpr (T::code == DT_F32) {
    st16_at(r, off, make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])));
    st16_at(r, off + 16u, make_uint4(__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]), __float_as_uint(y[7])));
  } else if constexpr (T::code == DT_BF16) {
    st16_at(r, off, make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])));
  } else {
    st16_at(r, off, make_uint4(pack_f16x2(y[0], y[1]), pack_f16x2(y[2], y[3]), pack_f16x2(y[4], y[5]), pack_f16x2(y[6], y[7])));
  }
}

// 8 float32 values stored in the output type dt at byte offset off (kOffNone: nothing stored)
__device__ __forceinline__ void store_out8_at(nf8_rsrc r, uint32_t off, const float (&y)[8], int dt) {
  if (dt == DT_F32) store_t8_at<F32>(r, off, y);
  else if (dt == DT_BF16) store_t8_at<BF16>(r, off, y);
  else store_t8_at<F16>(r, off, y);
}

// store 8 float32 values in the storage type T (used for dx)
template <class T> __device__ __forceinline__ void store_t8(void *base, int64_t elem, const float (&y)[8]) {
  store_out8(base, elem, y, T::code);
}

// ------------------------------------------------------------------------------------------
// FP8 (OCP E4M3 / E5M2). gfx950's v_cvt_pk_{fp8,bf8}_f32 convert to the OCP encodings with
// round-to-nearest-even; inputs are clamped to the largest finite value first so that
// out-of-range values saturate (the oracle's reading) rather than depend on the converter's
// overflow behaviour.
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ float fp8_max(int fmt) { return fmt == DT_E4M3 ? 448.0f : 57344.0f; }

// 8 float32 -> 8 FP8 codes packed little-endian in two dwords
__device__ __forceinline__ uint2 fp8_pack8(const float (&u)[8], int fmt) {
  const float m = fp8_max(fmt);
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_fmed3f(u[i], -m, m);
  // (the first conversion of each word keeps its destination's high half, which the second
  // overwrites: passing the first input's own bits there lets it convert in place, with no
  // copy of a zero into the destination)
  int w0, w1;
  const int k0 = (int)__float_as_uint(c[0]), k4 = (int)__float_as_uint(c[4]);
  if (fmt == DT_E4M3) {
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], k0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w0, true);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], k4, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], w1, true);
  } else {
    w0 = __builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], k0, false);
    w0 = __builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], w0, true);
    w1 = __builtin_amdgcn_cvt_pk_bf8_f32(c[4], c[5], k4, false);
    w1 = __builtin_amdgcn_cvt_pk_bf8_f32(c[6], c[7], w1, true);
  }
  return make_uint2((uint32_t)w0, (uint32_t)w1);
}

// MXFP8 shared exponent X of a block whose largest magnitude is `a` (float32, a >= 0):
// X = clamp(floor(log2 a) - emax, -127, 127); a zero or subnormal maximum gives -127.
// floor(log2 a) of a normal float32 is its unbiased exponent field.
__device__ __forceinline__ int mx_exponent(float a, int fmt, int ceil_rule) {
  // floor rule: X = floor(log2 a) - emax. Round-up rule (ceil_rule != 0): the smallest X with
  // a * 2^-X <= the format's largest finite value (1.75 * 2^emax for E4M3 and E5M2), i.e. one
  // more when a's significand exceeds 1.75 (binary32 fraction bits above 0x600000).
  const uint32_t b = __float_as_uint(a);
  const int emax = fmt == DT_E4M3 ? 8 : 15;
  const int ef = (int)((b >> 23) & 0xffu);
  int e = ef - 127 - emax;
  if (ceil_rule && ef != 0 && (b & 0x7fffffu) > 0x600000u) e += 1;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// 2^-X as float32 (X in [-127, 127] keeps the biased exponent 127 - X in [0, 254]; X = 127 gives
// 2^-127, a subnormal, built from the bit pattern)
__device__ __forceinline__ float exp2_neg(int x) {
  int b = 127 - x;
  return b > 0 ? __uint_as_float((uint32_t)b << 23) : __uint_as_float(0x00400000u);
}

// ------------------------------------------------------------------------------------------
// cross-lane reductions (wave64). Quad and row steps use DPP; the 16- and 32-lane steps use
// lane swaps. Every lane ends with the same value: each step combines a lane with a partner
// using a commutative operation.
// ------------------------------------------------------------------------------------------

#define NF8_DPP(ctrl) \
  __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), ctrl, 0xf, 0xf, false))

__device__ __forceinline__ float xor1(float v) { return NF8_DPP(0xB1); }   // quad_perm [1,0,3,2]
__device__ __forceinline__ float xor2(float v) { return NF8_DPP(0x4E); }   // quad_perm [2,3,0,1]
__device__ __forceinline__ float hmirror(float v) { return NF8_DPP(0x141); } // row_half_mirror
__device__ __forceinline__ float mirror(float v) { return NF8_DPP(0x140); }  // row_mirror
// The 16- and 32-lane steps use gfx950's lane-swap instructions (VALU, no LDS round trip):
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with the even rows of
// its second, v_permlane32_swap the upper half of the first with the lower half of the second.
// With both operands v, result[0] holds the even rows (lower half) and result[1] the odd rows
// (upper half) in both positions, so lane l's partner l ^ 16 (l ^ 32) is result[1] where l is in
// an even row (the lower half) and result[0] otherwise. Every lane of the wave must be active.
__device__ __forceinline__ float xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __uint_as_float((lane & 16) == 0 ? r[1] : r[0]);
}
__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __uint_as_float((lane & 32) == 0 ? r[1] : r[0]);
}
#undef NF8_DPP

__device__ __forceinline__ float wave_sum(float v) {
  v += xor1(v);
  v += xor2(v);
  v += hmirror(v);
  v += mirror(v);
  v += xor16(v);
  v += xor32(v);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor1(v));
  v = fmaxf(v, xor2(v));
  v = fmaxf(v, hmirror(v));
  v = fmaxf(v, mirror(v));
  v = fmaxf(v, xor16(v));
  v = fmaxf(v, xor32(v));
  return v;
}
// max over aligned groups of 4 lanes (one 32-element MX block = 4 strips)
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, xor1(v));
  v = fmaxf(v, xor2(v));
  return v;
}

// Partial statistics of a set of elements: count, mean and sum of squared deviations (the
// parallel-variance form that merges in one step). RMSNorm uses only `m2` as the sum of
// squares (n and mean unused).
struct Stats {
  float n, mean, m2;
};

// Chan et al. pairwise merge. Callers always pass the partner from the lower lane / wave /
// workgroup as `a`, so both partners compute bit-identical results. Branch-free: the weight
// b.n / n is taken with the hardware reciprocal, and an empty side leaves the other unchanged.
__device__ __forceinline__ Stats chan_merge(const Stats &a, const Stats &b) {
  const float n = a.n + b.n;
  const float d = b.mean - a.mean;
  const float fb = b.n * __builtin_amdgcn_rcpf(n);
  Stats r;
  r.n = n;
  r.mean = fmaf(d, fb, a.mean);
  r.m2 = a.m2 + b.m2 + d * d * (a.n * fb);
  const bool a_only = b.n == 0.0f, b_only = a.n == 0.0f;
  r.mean = a_only ? a.mean : (b_only ? b.mean : r.mean);
  r.m2 = a_only ? a.m2 : (b_only ? b.m2 : r.m2);
  return r;
}

// the value of `v` in the wave's first active lane (lane 0 where every lane is active)
__device__ __forceinline__ float first_lane(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// LayerNorm partial statistics taken relative to a shift K (the first element of the row
// piece a wave holds): sums of x - K instead of x, so that a row whose values share a large
// common part (x = 1000 + 0.01 * noise) keeps its deviations; x - K is exact for values
// within a factor of two of K. `s.mean` is relative to `k`.
struct ShiftedStats {
  Stats s;
  float k;
};
// `o` moved into the frame of shift `k`: its mean relative to k is (o.k - k) + o.s.mean, where
// o.k - k is exact when the shifts are close and otherwise small against the deviations
__device__ __forceinline__ Stats in_frame(const ShiftedStats &o, float k) {
  return Stats{o.s.n, (o.k - k) + o.s.mean, o.s.m2};
}

__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// wave-wide Chan merge; partner order fixed by lane position
__device__ __forceinline__ Stats wave_merge(Stats s) {
  const int lane = lane_id();
#define NF8_STEP(FN, LOW)                                                              \
  {                                                                                    \
    const Stats o{FN(s.n), FN(s.mean), FN(s.m2)};                                      \
    const bool lo = (LOW);                                                             \
    s = chan_merge(Stats{lo ? s.n : o.n, lo ? s.mean : o.mean, lo ? s.m2 : o.m2},       \
                   Stats{lo ? o.n : s.n, lo ? o.mean : s.mean, lo ? o.m2 : s.m2});      \
  }
  NF8_STEP(xor1, (lane & 1) == 0)
  NF8_STEP(xor2, (lane & 2) == 0)
  NF8_STEP(hmirror, (lane & 7) < 4)
  NF8_STEP(mirror, (lane & 15) < 8)
  NF8_STEP(xor16, (lane & 16) == 0)
  NF8_STEP(xor32, (lane & 32) == 0)
#undef NF8_STEP
  return s;
}

// ------------------------------------------------------------------------------------------
// cross-workgroup synchronisation through the workspace header
//
// gfx950 keeps one L2 per XCD and agent-scope fences write back / invalidate the whole L2, so
// the exchange avoids them: every word that crosses workgroups is written and read with
// agent-scope atomic operations (cache-coherent at device scope), and ordering between a
// workgroup's data writes and its counter update is enforced with a wait for outstanding
// memory operations plus a workgroup-scope fence.
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t max_dev(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t xchg_dev(uint32_t *p, uint32_t v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void or_dev(uint32_t *p, uint32_t v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// wait until this wave's outstanding vector-memory operations have completed, then order
// later memory operations after them (workgroup scope: no cache maintenance)
__device__ __forceinline__ void vmem_drain() {
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));  // vmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
}

__device__ __forceinline__ void st_dev64(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tagged(float v, uint32_t tag) {
  return ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
}
// the tag of the launch that observed `epoch` at its start (never 0)
__device__ __forceinline__ uint32_t epoch_tag(uint32_t epoch) { return epoch == 0xffffffffu ? 1u : epoch + 1u; }

// Value of a tagged word once it carries `tag`. Polls; after kSpinLimitTicks it sets bit 0 of
// *err and returns what it last read.
__device__ __forceinline__ float wait_tagged(const uint64_t *p, uint32_t tag, uint32_t *err) {
  uint64_t v = ld_dev64(p);
  if ((uint32_t)(v >> 32) == tag) return __uint_as_float((uint32_t)v);
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    v = ld_dev64(p);
    if ((uint32_t)(v >> 32) == tag) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimitTicks) {
      or_dev(err, 1u);
      break;
    }
  }
  return __uint_as_float((uint32_t)v);
}


// ------------------------------------------------------------------------------------------
// launch completion without a hot spot: workgroup g counts itself in group g / 64; the
// workgroup completing a group counts the group in kWsDone. Exactly one workgroup -- the last
// to finish -- sees both counters complete. Call from every thread after all of the
// workgroup's cross-workgroup results are stored (after vmem_drain); returns the same answer
// in every thread of the workgroup.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ bool finish_workgroup(uint32_t *ws, uint32_t *lds_flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int g = blockIdx.x / kWsGroupSize;
    const int ngroups = ((int)gridDim.x + kWsGroupSize - 1) / kWsGroupSize;
    const int rem = (int)gridDim.x - g * kWsGroupSize;
    const int gsize = rem < kWsGroupSize ? rem : kWsGroupSize;
    bool last = false;
    if (add_dev(ws + kWsGroup0 + g, 1u) == (uint32_t)(gsize - 1))
      last = add_dev(ws + kWsDone, 1u) == (uint32_t)(ngroups - 1);
    *lds_flag = last ? 1u : 0u;
  }
  __syncthreads();
  return *lds_flag != 0u;
}

// this workgroup's amax entry, tagged with its launch
__device__ __forceinline__ void publish_amax(uint32_t *ws, float a, uint32_t tag) {
  st_dev64(reinterpret_cast<uint64_t *>(ws + kWsAmax0) + blockIdx.x, tagged(a, tag));
}

// max over the per-workgroup amax entries [0, n) (all threads of the last workgroup). Each
// thread loads a batch of 8 entries before it looks at any of them, so a launch with a few
// thousand workgroups costs one round trip rather than one per entry; only an entry whose tag
// is not yet this launch's is polled again.
__device__ __forceinline__ float gather_amax(uint32_t *ws, int n, float *lds_red, uint32_t tag) {
  constexpr int B = 8;
  const uint64_t *parts = reinterpret_cast<const uint64_t *>(ws + kWsAmax0);
  const int nt = (int)blockDim.x;
  float a = 0.0f;
  for (int i0 = (int)threadIdx.x; i0 < n; i0 += B * nt) {
    uint64_t v[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = i0 + j * nt;
      v[j] = ld_dev64(parts + (i < n ? i : 0));  // (an index past the end reloads entry 0, unused)
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = i0 + j * nt;
      if (i < n) {
        const float x = (uint32_t)(v[j] >> 32) == tag ? __uint_as_float((uint32_t)v[j])
                                                       : wait_tagged(parts + i, tag, ws + kWsError);
        a = fmaxf(a, x);
      }
    }
  }
  a = wave_max(a);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds_red[w] = a;
  __syncthreads();
  float t = 0.0f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t = fmaxf(t, lds_red[i]);
  return t;
}

// re-zero the completion counters and advance the epoch (all threads of the last workgroup)
__device__ __forceinline__ void reset_completion(uint32_t *ws) {
  const int ngroups = ((int)gridDim.x + kWsGroupSize - 1) / kWsGroupSize;
  for (int i = threadIdx.x; i < ngroups; i += blockDim.x) xchg_dev(ws + kWsGroup0 + i, 0u);
  if (threadIdx.x == 0) {
    xchg_dev(ws + kWsDone, 0u);
    add_dev(ws + kWsEpoch, 1u);
  }
}

// epoch of the current launch (read by thread 0 at the start; broadcast through LDS)
__device__ __forceinline__ uint32_t read_epoch(uint32_t *ws, uint32_t *lds) {
  if (threadIdx.x == 0) *lds = ld_dev_u32(ws + kWsEpoch);
  __syncthreads();
  return *lds;
}

}  // namespace nf8
