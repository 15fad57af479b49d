// fwd_split.hip -- LayerNorm / RMSNorm forward for long rows, each row split over S workgroups
// whose weight slices stay in LDS.
//
// [XLA-Norm] = "Implementation: NVIDIA TransformerEngine JAX XLA Normalization";
// [NVRTC-PR] = "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request).
// [NVRTC-PR] Greptile Summary and Flowchart: rows too long for one CTA are split over several
// CTAs that combine their partial statistics through a workspace. [XLA-Norm] I/O Contract: the
// forward's outputs y, mu (LayerNorm) and rsigma.
//
// A row of H elements is cut into S = ceil(H / W) slices. A workgroup owns one slice of every row
// of its row group and loads the slice's gamma / beta (float32, 1 + gamma when zero-centred)
// once, then walks its rows, so no weight is read again from the caches per row (a 65536-element
// row re-read 512 KB of weights per row through the L2 in the one-workgroup-per-row layout).
// Lane t holds the strips of columns 8 (t + NT k), k < KC. Three shapes: 16 waves x 2 strips
// (W = 16384) with both weight arrays in LDS (128 KB for LayerNorm) and four rows in flight; and,
// for 16-bit input, 8 waves x 8 strips (W = 32768) with gamma in registers (64 per lane), beta in
// LDS (128 KB) and three rows in flight, or 8 waves x 4 strips (W = 16384) with gamma in
// registers (32 per lane), beta in LDS (64 KB) and four rows in flight.
//
// Per row: every wave reduces its elements of the slice (1024, 2048 or 4096; LayerNorm: deviations
// from the wave's plain mean estimate, so that a large common part of the row costs no
// precision), the waves' partials are merged through LDS in wave order, and the slice's partial is published to the
// workspace as tagged 64-bit words {value, launch tag}. Each workgroup then polls the S slices'
// words of the row and merges them in slice order, so all S workgroups obtain identical
// statistics. Four rows are in flight: row j + 3 is loading and row j + 2 publishes its partial
// while row j is normalised with its partners' words, which were published two rows earlier and
// loaded one row earlier, so the exchange overlaps the loads of the next rows. With three rows
// in flight (the 32768-column shape, whose registers hold 64 gamma values) row j + 2 loads and
// row j + 1 publishes while row j is normalised: each stage has one row's time to land.
//
// Group membership comes from tickets taken at start (group = ticket / S, slice = ticket % S):
// every ticket is held by a running workgroup, so a workgroup only waits on workgroups that are
// running or can still start; every wait has the 2 s limit of wait_tagged. The workgroup that
// finishes last re-zeroes the ticket counter and advances the launch epoch.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nf8 {

template <int NORM, class IN, int SH>
__global__ __launch_bounds__(kSplitShapes[SH].threads) void fwd_split_kernel(FwdSplitParams sp) {
  constexpr int NT = kSplitShapes[SH].threads;
  constexpr int KC = kSplitShapes[SH].strips;
  constexpr int W = (int)kSplitShapes[SH].cols();  // slice width (elements)
  constexpr bool WREG = kSplitShapes[SH].wreg != 0; // gamma in registers, beta in LDS
  constexpr int DEPTH = kSplitShapes[SH].depth;     // rows in flight
  static_assert(DEPTH == 3 || DEPTH == 4, "split pipeline depth");
  constexpr int NW = NORM == NT_LAYERNORM ? 2 : 1;  // weight arrays
  constexpr int NV = NORM == NT_LAYERNORM ? 3 : 1;  // tagged words per slice partial
  constexpr int NWAVE = NT / 64;
  const FwdRowParams &p = sp.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t H = p.hidden;
  const int64_t N = p.rows;
  const int S = sp.S;

  // LDS weights: [gamma][beta] (shape 0) or [beta] (register gamma; LayerNorm)
  constexpr int WL_FLOATS = WREG ? (NORM == NT_LAYERNORM ? W : 1) : NW * W;
  constexpr int BETA_OFF = WREG ? 0 : W;
  __shared__ __align__(16) float wlds[WL_FLOATS];
  __shared__ ShiftedStats wpart[2][NWAVE];
  __shared__ uint32_t s_ticket, s_epoch, s_last;

  if (tid == 0) {
    s_epoch = ld_dev_u32(p.ws + kWsEpoch);
    s_ticket = add_dev(p.ws + kWsTicket0, 1u);
  }
  __syncthreads();
  const uint32_t tag = epoch_tag(s_epoch);
  const int ticket = __builtin_amdgcn_readfirstlane((int)s_ticket);  // (scalar: so are the row and slice indices)
  const int group = ticket / S;
  const int slice = ticket - group * S;
  const int ngroups = (int)gridDim.x / S;
  const int64_t c0 = (int64_t)slice * W;
  const int cols = (int)(H - c0 < W ? H - c0 : W);  // columns of this slice

  // ---- the slice's weights, once
  float gr[WREG ? KC : 1][8];  // register gamma (shape 1): strip k's 8 weights, zero past the slice
  if constexpr (WREG) {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int c = 8 * (tid + NT * k);
      if (c < cols) {
        load_w8(gr[k], p.gamma, c0 + c, p.w_dtype);
        if (p.zero_centered) {
#pragma unroll
          for (int i = 0; i < 8; ++i) gr[k][i] += 1.0f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) gr[k][i] = 0.0f;
      }
    }
  }
  for (int c = 8 * tid; c < cols; c += 8 * NT) {
    float w[8];
    if constexpr (!WREG) {
      load_w8(w, p.gamma, c0 + c, p.w_dtype);
      if (p.zero_centered) {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] += 1.0f;
      }
      float4 *d = reinterpret_cast<float4 *>(wlds + c);
      d[0] = make_float4(w[0], w[1], w[2], w[3]);
      d[1] = make_float4(w[4], w[5], w[6], w[7]);
    }
    if constexpr (NORM == NT_LAYERNORM) {
      load_w8(w, p.beta, c0 + c, p.w_dtype);
      float4 *e = reinterpret_cast<float4 *>(wlds + BETA_OFF + c);
      e[0] = make_float4(w[0], w[1], w[2], w[3]);
      e[1] = make_float4(w[4], w[5], w[6], w[7]);
    }
  }

  bool cv[KC];
  float n_in = 0.0f;
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    cv[k] = 8 * (tid + NT * k) < cols;
    n_in += cv[k] ? 8.0f : 0.0f;
  }
  const float n_w = wave_sum(n_in);  // this wave's elements of the slice
  const float inv_nw = 1.0f / fmaxf(n_w, 1.0f);
  const float inv_h = 1.0f / (float)H;
  uint32_t *const err = p.ws + kWsError;
  __syncthreads();  // weights staged

  // rows of this group: group, group + ngroups, ... (nr of them)
  const int64_t nr = group < N ? (N - group + ngroups - 1) / ngroups : 0;
  auto row_of = [&](int64_t j) { return group + j * ngroups; };

  typedef Strip<IN> RowBuf[KC];
  // unconditional loads: a row past the group's last reads row 0, a strip past the slice reads
  // the slice's first strip (masked where used)
  auto load_row = [&](RowBuf &b, int64_t j) {
    const int64_t r = j < nr ? row_of(j) : 0;
#pragma unroll
    for (int k = 0; k < KC; ++k) load_strip<IN>(b[k], p.x, r * H + c0 + (cv[k] ? 8 * (tid + NT * k) : 0));
  };
  auto part_of = [&](int64_t r) { return sp.partials + r * (int64_t)S * NV; };

  // ---- statistics of row j's slice, published (every wave takes part: one barrier)
  auto stats_publish = [&](RowBuf &b, int64_t j) {
    if (cols != W) {
#pragma unroll
      for (int k = 0; k < KC; ++k) mask_strip<IN>(b[k], cv[k]);
    }
    ShiftedStats ws{Stats{0.0f, 0.0f, 0.0f}, 0.0f};
    if constexpr (NORM == NT_LAYERNORM) {
      float sa = 0.0f;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xv[8];
        strip_to_f32<IN>(b[k], xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) sa += xv[i];
      }
      // the wave's shift, rounded once (readfirstlane keeps a product from being fused into
      // each x - K)
      const float K = first_lane(wave_sum(sa) * inv_nw);
#pragma unroll
      for (int k = 0; k < KC; ++k) opaque<IN>(b[k]);  // converted again, not kept as floats
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xv[8];
        strip_to_f32<IN>(b[k], xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float d = cv[k] ? xv[i] - K : 0.0f;
          s1 += d;
          s2 = fmaf(d, d, s2);
        }
      }
      const float t1 = wave_sum(s1), t2 = wave_sum(s2);
      const float m = t1 * inv_nw;
      ws = ShiftedStats{Stats{n_w, m, fmaxf(fmaf(-t1, m, t2), 0.0f)}, K};
    } else {
      float q = 0.0f;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float xv[8];
        strip_to_f32<IN>(b[k], xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) q = fmaf(xv[i], xv[i], q);  // masked strips are zero
      }
      ws.s.m2 = wave_sum(q);
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) opaque<IN>(b[k]);  // (the row is converted again in finish)
    if (lane == 0) wpart[j & 1][wave] = ws;
    __syncthreads();
    if (wave == 0 && j < nr) {
      Stats st = wpart[j & 1][0].s;
      const float k0 = wpart[j & 1][0].k;
#pragma unroll 1
      for (int w = 1; w < NWAVE; ++w) {  // (not unrolled: the partials read ahead would take 4 registers each)
        const ShiftedStats o = wpart[j & 1][w];
        if constexpr (NORM == NT_LAYERNORM) st = chan_merge(st, in_frame(o, k0));
        else st.m2 += o.s.m2;
      }
      uint64_t *dst = part_of(row_of(j)) + slice * NV;
      if constexpr (NORM == NT_LAYERNORM) {
        const float v = lane == 0 ? st.mean : (lane == 1 ? st.m2 : k0);
        if (lane < NV) st_dev64(dst + lane, tagged(v, tag));
      } else {
        if (lane == 0) st_dev64(dst, tagged(st.m2, tag));
      }
    }
  };

  // The S slices' words of a row are loaded one row ahead of their use, before the stores of
  // the row in between: loads and stores retire in issue order, so a word loaded after a row's
  // stores (or after the next row's prefetch) could only be used once those had completed.
  auto poll_issue = [&](int64_t j) -> uint64_t {
    const uint64_t *pr = part_of(j < nr ? row_of(j) : 0);
    return lane < S * NV ? ld_dev64(pr + lane) : 0ull;
  };

  // ---- row j: the S partials (loaded as pv), merged in slice order; then the next row's words
  // are loaded, and the slice is normalised and stored
  auto finish = [&](RowBuf &b, int64_t j, uint64_t &pv) {
    const int64_t r = row_of(j);
    float v = __uint_as_float((uint32_t)pv);
    if (lane < S * NV && (uint32_t)(pv >> 32) != tag) v = wait_tagged(part_of(r) + lane, tag, err);
    float mu = 0.0f, rs;
    if constexpr (NORM == NT_LAYERNORM) {
      auto word = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
      const float k0 = word(2);
      Stats acc{(float)(H < W ? H : W), word(0), word(1)};
      for (int s = 1; s < S; ++s) {
        const int64_t left = H - (int64_t)s * W;
        const ShiftedStats o{Stats{(float)(left < W ? left : W), word(3 * s), word(3 * s + 1)}, word(3 * s + 2)};
        acc = chan_merge(acc, in_frame(o, k0));
      }
      mu = k0 + acc.mean;
      rs = __builtin_amdgcn_rsqf(acc.m2 * inv_h + p.eps);
    } else {
      float q = 0.0f;
      for (int s = 0; s < S; ++s)
        q += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), s));
      rs = __builtin_amdgcn_rsqf(q * inv_h + p.eps);
    }
    pv = poll_issue(j + 1);
    if (slice == 0 && tid == 0) {
      if (p.rsigma) p.rsigma[r] = rs;
      if constexpr (NORM == NT_LAYERNORM) {
        if (p.mu) p.mu[r] = mu;
      }
    }
    // (the row's y stores are issued on every path: buffer stores whose offset is moved past
    // the slice's end where a lane has nothing to write; a path on which a strip's store was
    // skipped would make the next wait for an earlier load drain every access in flight)
    const uint32_t ob = p.out_dtype == DT_F32 ? 4u : 2u;
    const nf8_rsrc ry = make_rsrc(static_cast<char *>(p.y) + (r * H + c0) * ob, (uint32_t)cols * ob);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int c = 8 * (tid + NT * k);
      float xv[8], y[8], gk[8];
      strip_to_f32<IN>(b[k], xv);
      if constexpr (WREG) {
#pragma unroll
        for (int i = 0; i < 8; ++i) gk[i] = gr[k][i];
      } else {
        const float4 *g4 = reinterpret_cast<const float4 *>(wlds + c);
        const float4 ga = g4[0], gb = g4[1];
        gk[0] = ga.x; gk[1] = ga.y; gk[2] = ga.z; gk[3] = ga.w;
        gk[4] = gb.x; gk[5] = gb.y; gk[6] = gb.z; gk[7] = gb.w;
      }
      if constexpr (NORM == NT_LAYERNORM) {
        const float4 *b4 = reinterpret_cast<const float4 *>(wlds + BETA_OFF + c);
        const float4 ba = b4[0], bb = b4[1];
        const float bk[8] = {ba.x, ba.y, ba.z, ba.w, bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = fmaf((xv[i] - mu) * rs, gk[i], bk[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = (xv[i] * rs) * gk[i];
      }
      store_out8_at(ry, cv[k] ? (uint32_t)c * ob : kOffNone, y, p.out_dtype);
      __builtin_amdgcn_sched_barrier(0);  // one strip's weights and values live at a time
    }
  };

  if constexpr (DEPTH == 4) {
    // four row buffers in turn: row j + 3 loads while row j + 2 is reduced and published and
    // row j finishes with the words loaded one row earlier (two rows after their publication)
    RowBuf A, B, C, D;
    load_row(A, 0);
    load_row(B, 1);
    load_row(C, 2);
    stats_publish(A, 0);
    stats_publish(B, 1);
    uint64_t pv = poll_issue(0);
    for (int64_t j = 0; j < nr; j += 4) {
      load_row(D, j + 3);
      stats_publish(C, j + 2);
      finish(A, j, pv);
      if (j + 1 >= nr) break;
      load_row(A, j + 4);
      stats_publish(D, j + 3);
      finish(B, j + 1, pv);
      if (j + 2 >= nr) break;
      load_row(B, j + 5);
      stats_publish(A, j + 4);
      finish(C, j + 2, pv);
      if (j + 3 >= nr) break;
      load_row(C, j + 6);
      stats_publish(B, j + 5);
      finish(D, j + 3, pv);
    }
  } else {
    // three row buffers in turn: row j + 2 loads while row j + 1 is reduced and published and
    // row j finishes with the words published one row earlier
    RowBuf A, B, C;
    load_row(A, 0);
    load_row(B, 1);
    stats_publish(A, 0);
    uint64_t pv = poll_issue(0);
    for (int64_t j = 0; j < nr; j += 3) {
      load_row(C, j + 2);
      stats_publish(B, j + 1);
      finish(A, j, pv);
      if (j + 1 >= nr) break;
      load_row(A, j + 3);
      stats_publish(C, j + 2);
      finish(B, j + 1, pv);
      if (j + 2 >= nr) break;
      load_row(B, j + 4);
      stats_publish(A, j + 3);
      finish(C, j + 2, pv);
    }
  }

  // ---- end of launch: the last workgroup re-zeroes the ticket counter and advances the epoch
  vmem_drain();
  if (finish_workgroup(p.ws, &s_last)) {
    if (tid == 0) xchg_dev(p.ws + kWsTicket0, 0u);
    vmem_drain();
    __syncthreads();
    reset_completion(p.ws);
  }
}

template <int NORM>
static const void *pick_split_in(int in_dtype, int shape) {
  if (shape == 1 || shape == 2) {  // (16-bit input only: float32 rows would not fit beside gamma)
    switch (in_dtype) {
      case DT_BF16: return shape == 1 ? (const void *)fwd_split_kernel<NORM, BF16, 1> : (const void *)fwd_split_kernel<NORM, BF16, 2>;
      case DT_F16: return shape == 1 ? (const void *)fwd_split_kernel<NORM, F16, 1> : (const void *)fwd_split_kernel<NORM, F16, 2>;
      default: return nullptr;
    }
  }
  if (shape != 0) return nullptr;
  switch (in_dtype) {
    case DT_F32: return (const void *)fwd_split_kernel<NORM, F32, 0>;
    case DT_BF16: return (const void *)fwd_split_kernel<NORM, BF16, 0>;
    case DT_F16: return (const void *)fwd_split_kernel<NORM, F16, 0>;
    default: return nullptr;
  }
}

const void *fwd_split_kernel_ptr(int norm, int in_dtype, int shape) {
  return norm == NT_LAYERNORM ? pick_split_in<NT_LAYERNORM>(in_dtype, shape)
                              : pick_split_in<NT_RMSNORM>(in_dtype, shape);
}

}  // namespace nf8
