// fwd_col.hip -- LayerNorm / RMSNorm forward with a columnwise (transposed) FP8 output whose
// column segments are written as whole 128-byte lines.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization".
// [XLA-Norm] Description: besides the rowwise FP8 output, an optional columnwise output with
// its own scale_inv, for delayed per-tensor scaling and for MXFP8 block scaling; the norm and
// the quantisation happen in one kernel launch. Here the columnwise tensor is [hidden, rows]
// (the transpose), and for MXFP8 each columnwise block is 32 consecutive rows of one column.
//
// Why 128-row tiles: a column of the transposed output is contiguous along rows, so a tile of
// R rows writes R bytes per column. On MI355X, column pieces shorter than a 128-byte line are
// not merged on their way to HBM (a 32-byte piece costs close to a whole line of write
// traffic), so a workgroup owns 128 rows and writes each column segment as one line.
//
// Work split: a workgroup of 16 waves owns a tile of 128 rows x 512 columns; wave w owns rows
// [8w, 8w + 8) of the tile and lane l the 8 columns [8l, 8l + 8), so every lane holds an 8 x 8
// block. S = ceil(hidden / 512) tiles make one band of 128 full rows; the S workgroups that
// hold them combine per-row partial statistics through tagged workspace words. FP8 codes are
// transposed in registers (4 x 4 byte blocks), staged in LDS as [column][128 rows] (each
// column's 8-row pieces XOR-swizzled so neighbouring columns use different banks), and stored
// so that 8 consecutive lanes write one column's 128-byte line with 16-byte stores.
//
// Scheduling and progress: the persistent grid takes tiles from per-class ticket counters
// (ticket t = band t / S, slice t % S). A workgroup publishes a tile's statistics right after
// loading it and before it waits for anything; it takes its next ticket only after that wait
// is over, and loads the next tile while it writes the current tile's outputs. Hence every
// ticket handed out is published without any wait in between, a wait can only be on bands
// whose tickets are all handed out or on the newest band, and the newest band is completed by
// the workgroups that are not waiting (the planner launches at least 2S per class).
#include "device_common.hpp"
#include "kernels.hpp"

namespace nf8 {

namespace {

constexpr int kColRows = 128;  // rows per tile (one 128-byte line per column)
constexpr int kColWaves = 16;
constexpr int kColRW = 8;      // rows per wave
constexpr int kColCW = 512;    // columns per tile
constexpr int kStageBytes = kColCW * kColRows;

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
  return col * kColRows + 8 * (piece ^ ((col >> 3) & 15));
}

}  // namespace

template <int NORM, class IN, int MODE>
__global__ __launch_bounds__(1024) void fwd_col_kernel(FwdBandParams bp) {
  static_assert(MODE == MODE_DELAYED || MODE == MODE_MX, "columnwise output is FP8");
  constexpr int RW = kColRW;
  constexpr int NV = NORM == NT_LAYERNORM ? 2 : 1;
  constexpr uint32_t ES = IN::bytes;
  // the next tile is loaded during the current tile's outputs when both fit in registers
  constexpr bool PF = sizeof(Strip<IN>) == 16;
  const FwdRowParams &p = bp.f;
  // tid and lane are re-made opaque at the top of every tile so that the compiler recomputes
  // the per-lane addresses there instead of keeping dozens of them live across the loop
  int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int S = bp.S;
  const int64_t H = p.hidden;
  const int64_t N = p.rows;
  const int fmt = p.out_dtype;

  // staging buffer: transposed codes; during the statistics exchange it holds the fetched
  // partials as float[16 waves][8 rows][S][NV] (64 KB for S = 64)
  __shared__ __align__(16) uint8_t stage[kStageBytes];
  __shared__ __align__(16) float colmax[MODE == MODE_MX ? kColWaves : 1][MODE == MODE_MX ? kColCW : 1];
  __shared__ uint8_t colx[MODE == MODE_MX ? 4 : 1][MODE == MODE_MX ? kColCW : 1];
  __shared__ int s_next;
  __shared__ uint32_t s_last, s_epoch;
  __shared__ float wred[kColWaves];
  float *const xpart = reinterpret_cast<float *>(stage) + wave * RW * S * NV;

  const int ncls = bp.classes;
  const int cls = (int)(blockIdx.x % ncls);
  const int wpc = (int)gridDim.x / ncls;
  const int lwg = (int)blockIdx.x / ncls;
  const int64_t b0 = bp.bands * cls / ncls;
  const int64_t b1 = bp.bands * (cls + 1) / ncls;
  const int ntiles = (int)((b1 - b0) * S);
  uint32_t *const ticket = S > 1 ? p.ws + kWsTicket0 + cls : nullptr;
  const bool coordinated = MODE == MODE_DELAYED || S > 1;
  const uint32_t tag = coordinated ? epoch_tag(read_epoch(p.ws, &s_epoch)) : 0u;

  // next tile of this workgroup (all threads call it; with S > 1 it contains a barrier)
  auto take_ticket = [&](int prev) -> int {
    if (S == 1) return prev < 0 ? lwg : prev + wpc;
    if (tid == 0) s_next = (int)add_dev(ticket, 1u);
    __syncthreads();
    return s_next;
  };

  // Offsets inside a tile fit in 32 bits (128 rows of at most 2^15 elements); every tile
  // address is a wave-uniform 64-bit base plus a 32-bit per-lane offset.
  const uint32_t row_bytes = (uint32_t)H * ES;

  auto load_tile = [&](Strip<IN> (&xs)[RW], int t) {
    const int tb = t / S;
    const int sl = t - tb * S;
    const int64_t band = b0 + tb;
    const int64_t r0 = band * kColRows + RW * wave;
    const bool cv = (int64_t)sl * kColCW + 8 * lane < H;
    const char *xt = static_cast<const char *>(p.x) + (band * kColRows * H + (int64_t)sl * kColCW) * ES;
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      if (t < ntiles && r0 + j < N && cv) {
        const uint32_t off = (uint32_t)(wave * RW + j) * row_bytes + 8u * ES * (uint32_t)lane;
        const uint4 *src = reinterpret_cast<const uint4 *>(xt + off);
#pragma unroll
        for (int i = 0; i < (int)(sizeof(Strip<IN>) / 16); ++i) xs[j].v[i] = src[i];
      } else {
        zero_strip<IN>(xs[j]);
      }
    }
  };
  // wave-merged partial statistics of the wave's 8 rows over the tile's columns (every lane
  // ends with the same values); RMSNorm keeps only the sum of squares
  auto tile_stats = [&](const Strip<IN> (&xs)[RW], int t, Stats (&st)[RW]) {
    if constexpr (NORM == NT_LAYERNORM) {
      const int tb = t / S;
      const int sl = t - tb * S;
      const int64_t r0 = (b0 + tb) * kColRows + RW * wave;
      const bool cv = t < ntiles && (int64_t)sl * kColCW + 8 * lane < H;
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        float xv[8];
        strip_to_f32<IN>(xs[j], xv);
        const bool ok = cv && r0 + j < N;
        float sm = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sm += xv[i];
        const float m = ok ? sm * 0.125f : 0.0f;
        float q = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float d = xv[i] - m;
          q = fmaf(d, d, q);
        }
        st[j] = wave_merge(Stats{ok ? 8.0f : 0.0f, m, ok ? q : 0.0f});
      }
    } else {
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        float xv[8];
        strip_to_f32<IN>(xs[j], xv);
        float q = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) q = fmaf(xv[i], xv[i], q);
        st[j] = Stats{0.0f, 0.0f, wave_sum(q)};
      }
    }
  };
  auto publish = [&](const Stats (&st)[RW], int t) {
    if (S == 1 || t >= ntiles) return;
    const int tb = t / S;
    const int sl = t - tb * S;
    uint64_t *part = bp.partials + ((b0 + tb) * S + sl) * (int64_t)kColRows * NV + (wave * RW) * NV;
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      if (lane == j) {
        if constexpr (NORM == NT_LAYERNORM) {
          st_dev64(part + j * NV, tagged(st[j].mean, tag));
          st_dev64(part + j * NV + 1, tagged(st[j].m2, tag));
        } else {
          st_dev64(part + j, tagged(st[j].m2, tag));
        }
      }
    }
  };

  float scale = 1.0f;
  if constexpr (MODE == MODE_DELAYED) scale = *p.scale;
  float amax_local = 0.0f;
  const float inv_h = 1.0f / (float)H;

  Strip<IN> cur[RW], nxt[RW];
  Stats st[RW];
  int tk = take_ticket(-1);
  load_tile(cur, tk);
  tile_stats(cur, tk, st);
  publish(st, tk);

  while (tk < ntiles) {
    asm volatile("" : "+v"(tid), "+v"(lane));
    const int tb = tk / S;
    const int slice = tk - tb * S;
    const int64_t band = b0 + tb;
    const int64_t cbase = (int64_t)slice * kColCW;
    const bool cv = cbase + 8 * lane < H;
    const int64_t rbase = band * kColRows + RW * wave;
    const int valid_rows = (int)(N - rbase < RW ? (N - rbase < 0 ? 0 : N - rbase) : RW);

    // ---- the band's statistics: each lane polls some (row, slice) entries of this wave's
    // rows into LDS, then lane j merges row j's S partials in slice order
    if (S > 1) {
      const uint64_t *bpart = bp.partials + band * S * (int64_t)kColRows * NV + (wave * RW) * NV;
      for (int e = lane; e < RW * S; e += 64) {
        const int j = e / S;
        const int sl = e - j * S;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          xpart[e * NV + v] = wait_tagged(bpart + (sl * kColRows + j) * NV + v, tag, p.ws + kWsError);
      }
      __syncthreads();
      Stats acc{0.0f, 0.0f, 0.0f};
      if (lane < RW) {
        for (int sl = 0; sl < S; ++sl) {
          const float *e = xpart + (lane * S + sl) * NV;
          if constexpr (NORM == NT_LAYERNORM) {
            const int64_t left = H - (int64_t)sl * kColCW;
            acc = chan_merge(acc, Stats{(float)(left < kColCW ? left : kColCW), e[0], e[1]});
          } else {
            acc.m2 += e[0];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        if constexpr (NORM == NT_LAYERNORM)
          st[j].mean = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acc.mean), j));
        st[j].m2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acc.m2), j));
      }
    }
    float mu[RW], rs[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      mu[j] = NORM == NT_LAYERNORM ? st[j].mean : 0.0f;
      rs[j] = 1.0f / sqrtf(st[j].m2 * inv_h + p.eps);
    }
    if (slice == 0 && lane < valid_rows) {
      float m = mu[0], r = rs[0];
#pragma unroll
      for (int j = 1; j < RW; ++j) {
        m = lane == j ? mu[j] : m;
        r = lane == j ? rs[j] : r;
      }
      if (p.rsigma) p.rsigma[rbase + lane] = r;
      if constexpr (NORM == NT_LAYERNORM) {
        if (p.mu) p.mu[rbase + lane] = m;
      }
    }

    // ---- next ticket (this workgroup waits for nothing more in this band); its loads stay in
    // flight while this tile's outputs are produced. With S > 1 the barrier inside also orders
    // the LDS partial reads above before the staging writes below.
    const int tn = take_ticket(tk);
    if constexpr (PF) load_tile(nxt, tn);

    const int64_t col = cbase + 8 * lane;
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
    auto yrow = [&](int j, float (&y)[8]) {
      float xv[8];
      strip_to_f32<IN>(cur[j], xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (NORM == NT_LAYERNORM) y[i] = fmaf((xv[i] - mu[j]) * rs[j], gk[i], bk[i]);
        else y[i] = (xv[i] * rs[j]) * gk[i];
      }
    };
    uint8_t *const yt = static_cast<uint8_t *>(p.y) + band * kColRows * H + cbase;

    // ---- MXFP8 columnwise scales: block = 32 rows = 4 waves
    float colf[8];
    if constexpr (MODE == MODE_MX) {
      float cm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        float y[8];
        yrow(j, y);
        if (j < valid_rows) {
#pragma unroll
          for (int i = 0; i < 8; ++i) cm[i] = fmaxf(cm[i], fabsf(y[i]));
        }
      }
      float4 *dst = reinterpret_cast<float4 *>(&colmax[wave][8 * lane]);
      dst[0] = make_float4(cm[0], cm[1], cm[2], cm[3]);
      dst[1] = make_float4(cm[4], cm[5], cm[6], cm[7]);
#pragma unroll
      for (int j = 0; j < RW; ++j) opaque<IN>(cur[j]);  // recompute y below, do not keep it
      __syncthreads();
      const int q = wave >> 2;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = 8 * lane + i;
        const float a = fmaxf(fmaxf(colmax[4 * q][c], colmax[4 * q + 1][c]), fmaxf(colmax[4 * q + 2][c], colmax[4 * q + 3][c]));
        const int X = mx_exponent(a, fmt);
        colf[i] = exp2_neg(X);
        if ((wave & 3) == 0) colx[q][c] = (uint8_t)(X + 127);
      }
    }

    // ---- codes: rowwise stores; columnwise codes transposed (4 rows at a time) into LDS
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint2 codes[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * h + jj;
        const bool ok = (j < valid_rows) && cv;
        const uint32_t yoff = (uint32_t)(wave * RW + j) * (uint32_t)H + 8u * (uint32_t)lane;
        float y[8];
        yrow(j, y);
        if constexpr (MODE == MODE_DELAYED) {
          float u[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            u[i] = y[i] * scale;
            if (ok) amax_local = fmaxf(amax_local, fabsf(y[i]));
          }
          codes[jj] = fp8_pack8(u, fmt);
          if (ok && bp.write_row) *reinterpret_cast<uint2 *>(yt + yoff) = codes[jj];
        } else {
          if (bp.write_row) {
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
              *reinterpret_cast<uint2 *>(yt + yoff) = c;
              if ((lane & 3) == 0) {
                uint8_t *sr = static_cast<uint8_t *>(p.scale_inv) + (rbase + j) * p.mx_cols + (cbase >> 5);
                sr[lane >> 2] = (uint8_t)(X + 127);
              }
            }
          }
          float u[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) u[i] = y[i] * colf[i];
          codes[jj] = fp8_pack8(u, fmt);
        }
      }
      uint32_t lo[4], hi[4];  // lo[i]: column i, hi[i]: column 4 + i; byte jj = row 4h + jj
      transpose4x4b(codes[0].x, codes[1].x, codes[2].x, codes[3].x, lo);
      transpose4x4b(codes[0].y, codes[1].y, codes[2].y, codes[3].y, hi);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint32_t *>(stage + stage_off(8 * lane + i, wave) + 4 * h) = i < 4 ? lo[i] : hi[i - 4];
    }
    __syncthreads();

    // ---- columnwise stores: thread (c, m) writes rows [16m, 16m + 16) of tile column c, so 8
    // consecutive lanes cover the column's 128 rows
    {
      const int64_t rows_here = N - band * kColRows;  // valid rows of this band (may be < 128)
      const bool full = rows_here >= kColRows && (N % 16) == 0;
      uint8_t *const yct = static_cast<uint8_t *>(bp.y_col) + cbase * N + band * kColRows;
      const int m = tid & 7;
#pragma unroll
      for (int pass = 0; pass < kColCW / 128; ++pass) {
        const int c = pass * 128 + (tid >> 3);
        if (cbase + c < H) {
          const int slot = (2 * m) ^ ((c >> 3) & 15);  // piece 2m; piece 2m + 1 is at slot ^ 1
          const uint2 a = *reinterpret_cast<const uint2 *>(stage + c * kColRows + 8 * slot);
          const uint2 b = *reinterpret_cast<const uint2 *>(stage + c * kColRows + 8 * (slot ^ 1));
          uint8_t *dst = yct + (int64_t)c * N + 16 * m;
          if (full) {
            *reinterpret_cast<uint4 *>(dst) = make_uint4(a.x, a.y, b.x, b.y);
          } else {
            const uint32_t w[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (16 * m + e < rows_here) dst[e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
          }
        }
      }
      if constexpr (MODE == MODE_MX) {
        // the band's (up to) four 32-row block exponents of each column
        if (tid < kColCW && cbase + tid < H) {
          uint8_t *dst = static_cast<uint8_t *>(bp.col_scale_inv) + (cbase + tid) * bp.mx_rows + 4 * band;
          const int64_t nb = (rows_here + 31) / 32;
          for (int q = 0; q < 4 && q < nb; ++q) dst[q] = colx[q][tid];
        }
      }
    }

    // ---- next tile: statistics published before this workgroup waits again
    if constexpr (PF) {
#pragma unroll
      for (int j = 0; j < RW; ++j) cur[j] = nxt[j];
    } else {
      load_tile(cur, tn);
    }
    tile_stats(cur, tn, st);
    publish(st, tn);
    __syncthreads();  // staging / colmax / colx are rewritten for the next tile
    tk = tn;
  }

  // ---- end of launch: amax publication and counter reset by the last workgroup
  if constexpr (MODE == MODE_DELAYED) {
    const float m = wave_max(amax_local);
    if (lane == 0) wred[wave] = m;
    __syncthreads();
    if (tid == 0) {
      float a = wred[0];
      for (int w = 1; w < kColWaves; ++w) a = fmaxf(a, wred[w]);
      publish_amax(p.ws, a, tag);
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

template <int NORM, class IN>
static const void *pick_col_mode(int mode) {
  switch (mode) {
    case MODE_DELAYED: return (const void *)fwd_col_kernel<NORM, IN, MODE_DELAYED>;
    case MODE_MX: return (const void *)fwd_col_kernel<NORM, IN, MODE_MX>;
    default: return nullptr;
  }
}

template <int NORM>
static const void *pick_col_in(int in_dtype, int mode) {
  switch (in_dtype) {
    case DT_F32: return pick_col_mode<NORM, F32>(mode);
    case DT_BF16: return pick_col_mode<NORM, BF16>(mode);
    case DT_F16: return pick_col_mode<NORM, F16>(mode);
    default: return nullptr;
  }
}

const void *fwd_col_kernel_ptr(int norm, int in_dtype, int mode) {
  return norm == NT_LAYERNORM ? pick_col_in<NT_LAYERNORM>(in_dtype, mode) : pick_col_in<NT_RMSNORM>(in_dtype, mode);
}

}  // namespace nf8
