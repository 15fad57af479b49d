/*
 * normfp8.h -- C ABI of the fused LayerNorm / RMSNorm + FP8 library for AMD MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [XLA-Norm]  "Implementation: NVIDIA TransformerEngine JAX XLA Normalization"
 *   [BwdAdd]    "Implementation: NVIDIA TransformerEngine Ops Fused Backward Add RMSNorm"
 *   [NVRTC-PR]  "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All functions are extern "C", thread-safe and non-blocking. They return NORM_OK (0) or
 *    a norm_status_t; norm_last_error() gives a message for the calling thread.
 *  - Arguments are validated on the host before anything is enqueued: on any error nothing
 *    has been enqueued on the stream.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream. Work is
 *    enqueued on that stream only. The library never synchronises, never allocates or frees
 *    device memory and never reads device memory on the host (norm_workspace_check excepted).
 *  - Tensors are device pointers to dense row-major storage. x-like tensors are [rows, hidden]
 *    with row stride `hidden` (1 <= hidden <= 2^24). Tensor pointers must be aligned to their
 *    element size and the workspace to 16 bytes. The vector kernels serve 16-byte-aligned
 *    tensors with hidden a multiple of 8 (rows up to 16384 elements in the backward); any other
 *    case goes to the general kernels ([NVRTC-PR] Greptile Summary: general variants beside the
 *    tuned ones), which compute the same results element by element, more slowly. The caller
 *    owns every buffer, including the workspace.
 *  - Element types are given by norm_dtype_t codes. Statistics (mu, rsigma) and the amax /
 *    scale / scale_inv scalars are always float32. rows == 0 is valid: row-indexed buffers
 *    (x, y, y_colwise, dy, dx, residual_dy, mu, rsigma, MXFP8 scale grids) may then be NULL;
 *    delayed scaling still writes updated_amax = *amax and scale_inv, and the backward
 *    writes zero weight gradients.
 *  - Workspace: the size comes from the *_workspace_size query for the same arguments. Every
 *    workspace begins with a NORM_WS_HEADER_BYTES synchronisation header that must be all
 *    zero before the workspace is first used (zero-fill it, or call norm_workspace_init once).
 *    Every call leaves the header zeroed again, so one workspace can serve any sequence of
 *    calls, of any shape, issued in order on one stream. Two calls that may run at the same
 *    time (different streams) must not share a workspace.
 */
#ifndef NORMFP8_H
#define NORMFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NORMFP8_ABI_VERSION 2
#define NORM_WS_HEADER_BYTES 16384

typedef enum {
  NORM_OK = 0,
  NORM_ERR_INVALID_ARG = 1,         /* NULL where a pointer is required, bad enum, negative size */
  NORM_ERR_UNSUPPORTED = 2,         /* valid request outside what this build implements */
  NORM_ERR_MISALIGNED = 3,          /* pointer not aligned to its element size (workspace: 16 bytes) */
  NORM_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace_bytes below the query's answer */
  NORM_ERR_HIP = 5                  /* a HIP runtime call failed (message has hipGetErrorString) */
} norm_status_t;

/* [XLA-Norm] Signature, I/O Contract: the norm type input selects LayerNorm or RMSNorm. */
typedef enum { NORM_LAYERNORM = 0, NORM_RMSNORM = 1 } norm_type_t;

/* [XLA-Norm] Signature: separate input, weight and output element types. */
typedef enum {
  NORM_F32 = 0,
  NORM_F16 = 1,
  NORM_BF16 = 2,
  NORM_FP8_E4M3 = 3, /* OCP E4M3 ("FN": bias 7, no inf, max 448) */
  NORM_FP8_E5M2 = 4  /* OCP E5M2 (bias 15, IEEE-style inf/NaN, max 57344) */
} norm_dtype_t;

/* [XLA-Norm] Description: delayed per-tensor scaling, MXFP8 block scaling, or no scaling. */
typedef enum {
  NORM_SCALING_NONE = 0,
  NORM_SCALING_DELAYED_TENSOR = 1,
  NORM_SCALING_MXFP8_1D32 = 2,     /* 32-element blocks, one E8M0 scale byte per block */
  NORM_SCALING_MXFP8_1D32_CEIL = 3 /* the same blocks, exponent rounded up: no element saturates */
} norm_scaling_t;

/* [XLA-Norm] Signature / Description: rowwise output with optional columnwise output. */
typedef enum {
  NORM_Q_ROWWISE = 1,
  NORM_Q_COLWISE = 2,
  NORM_Q_ROWWISE_COLWISE = 3,
  /* modifier, with NORM_Q_COLWISE: the columnwise output keeps the rowwise [rows, hidden] layout
     (codes of the columnwise quantisation in place, MXFP8 scales [ceil(rows/32), hidden]) */
  NORM_Q_COLWISE_ROWMAJOR = 4,
  /* modifier, MXFP8 only: E8M0 grids padded for consumers that read scales in whole tiles
     (see norm_fwd) */
  NORM_Q_SCALES_PADDED = 8
} norm_qlayout_t;

/*
 * norm_fwd_workspace_size -- bytes of workspace norm_fwd needs for these arguments.
 * [XLA-Norm] Description, Signature (forward workspace query: batch, hidden, the three element
 * types, norm type, scaling mode, zero-centred gamma, epsilon, SM margin, training flag).
 * `cu_margin` is the number of compute units the launch plan leaves free, as the pages' SM
 * margin. The answer depends only on the arguments (not on the device), so it can be taken
 * without a GPU. *bytes == 0 means workspace may be NULL.
 */
int norm_fwd_workspace_size(int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int out_dtype,
                            int norm_type, int scaling, int qlayout, int zero_centered_gamma,
                            float epsilon, int cu_margin, int is_training, size_t *bytes);

/*
 * norm_bwd_workspace_size -- bytes of workspace norm_bwd / norm_bwd_add need.
 * [XLA-Norm] Signature (backward workspace query); [NVRTC-PR] Flowchart (the backward keeps
 * per-workgroup weight-gradient partials for a finalize step). `with_add` selects norm_bwd_add.
 */
int norm_bwd_workspace_size(int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int norm_type,
                            int zero_centered_gamma, float epsilon, int cu_margin, int with_add,
                            size_t *bytes);

/*
 * norm_fwd -- normalise each row of x and store the output, optionally FP8-quantised, in one
 * kernel launch on `stream`. Columnwise layouts take one launch for RMSNorm with 16-bit input,
 * hidden a multiple of 512 and rows a multiple of 128 (x read once; the workgroups holding a
 * band of rows exchange their row sums through the workspace), and two otherwise (the row
 * statistics or rowwise codes first, then the columnwise codes). [XLA-Norm] Overview,
 * Description, Signature (NormForwardFFI argument list), I/O Contract.
 *
 *   x [rows, hidden] in_dtype; gamma [hidden] w_dtype; beta [hidden] w_dtype (LayerNorm only,
 *   must be NULL for RMSNorm).
 *   Statistics: mu [rows] (LayerNorm; NULL allowed) = row mean; rsigma [rows] (NULL allowed)
 *   = 1/sqrt(biased variance + epsilon) for LayerNorm, 1/sqrt(mean(x^2) + epsilon) for RMSNorm.
 *   Effective weight g = gamma, or 1 + gamma when zero_centered_gamma != 0.
 *   y_row = (x - mu) * rsigma * g + beta (LayerNorm) or x * rsigma * g (RMSNorm), in float32.
 *
 *   scaling == NORM_SCALING_NONE: y [rows, hidden] out_dtype (F32/F16/BF16), round-to-nearest-
 *     even of y_row. y_colwise, scale, amax, scale_inv, colwise_scale_inv, updated_amax unused
 *     (pass NULL). qlayout must be NORM_Q_ROWWISE.
 *   scaling == NORM_SCALING_DELAYED_TENSOR: out_dtype FP8_E4M3 or FP8_E5M2; scale, amax: device
 *     float32[1] inputs; codes = saturating nearest-even FP8 of y_row * scale. Rowwise codes in y
 *     [rows, hidden]; columnwise codes in y_colwise [hidden, rows] (the transpose). scale_inv and
 *     colwise_scale_inv (float32[1] each, for the layouts requested) receive 1/scale.
 *     updated_amax (float32[1], may alias amax) receives max(*amax, max |y_row|) over the tensor.
 *   scaling == NORM_SCALING_MXFP8_1D32: out_dtype FP8_E4M3 or FP8_E5M2; each block of 32
 *     consecutive elements (along a row for rowwise, along a column for columnwise; a final
 *     shorter block where the dimension is not a multiple of 32) shares the E8M0 scale
 *     2^X, X = clamp(floor(log2 amax_block) - emax, -127, 127) (emax 8 for E4M3, 15 for E5M2;
 *     X = -127 for an all-zero block); codes = saturating nearest-even FP8 of y_row * 2^-X.
 *     Rowwise: y [rows, hidden] codes, scale_inv = uint8 [rows, ceil(hidden/32)] bytes X+127.
 *     Columnwise: y_colwise [hidden, rows] codes, colwise_scale_inv = uint8
 *     [hidden, ceil(rows/32)]. scale, amax, updated_amax unused (NULL).
 *   scaling == NORM_SCALING_MXFP8_1D32_CEIL: as NORM_SCALING_MXFP8_1D32, except that X is the
 *     smallest integer with amax_block * 2^-X <= the format's largest finite value (448 for
 *     E4M3, 57344 for E5M2), clamped to [-127, 127], so no code saturates. The pages leave the
 *     exponent rule of their MXFP8 mode open; the floor rule is the default reading.
 *   With NORM_Q_COLWISE_ROWMAJOR added to a columnwise qlayout, y_colwise is [rows, hidden]
 *     (element (r, c) holds the code the transposed layout keeps at (c, r)) and the MXFP8
 *     colwise_scale_inv is uint8 [ceil(rows/32), hidden]; this build serves it for rows that a
 *     row layout covers (hidden <= 65536) and returns NORM_ERR_UNSUPPORTED otherwise.
 *   With NORM_Q_SCALES_PADDED added (MXFP8 only; for callers that hand the E8M0 grids to
 *     matrix-multiply kernels reading scales in whole tiles): in each grid the dimension that
 *     counts 32-element blocks is rounded up to a multiple of 4 and the other dimension to a
 *     multiple of 128, so scale_inv is [round_up(rows, 128), round_up(ceil(hidden/32), 4)],
 *     colwise_scale_inv [round_up(hidden, 128), round_up(ceil(rows/32), 4)], or with
 *     NORM_Q_COLWISE_ROWMAJOR [round_up(ceil(rows/32), 4), round_up(hidden, 128)]. The kernels
 *     write the logical region only; the padding keeps whatever the caller put there. The
 *     pages name no padded layout: this is a reading, its parity with the pages' system unpinned.
 *   The layout pointers not requested by qlayout must be NULL.
 *
 *   Errors: NORM_ERR_INVALID_ARG for NULL required pointers or bad codes; NORM_ERR_UNSUPPORTED
 *   for a dtype / layout combination this build does not implement; NORM_ERR_MISALIGNED;
 *   NORM_ERR_WORKSPACE_TOO_SMALL; NORM_ERR_HIP if the launch fails.
 */
int norm_fwd(void *stream, const void *x, const void *gamma, const void *beta, const float *scale,
             const float *amax, void *y, void *y_colwise, float *mu, float *rsigma, void *scale_inv,
             void *colwise_scale_inv, float *updated_amax, void *workspace, size_t workspace_bytes,
             int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int out_dtype, int norm_type,
             int scaling, int qlayout, int zero_centered_gamma, float epsilon, int cu_margin);

/*
 * norm_bwd -- LayerNorm / RMSNorm backward. [XLA-Norm] Description (backward dispatch);
 * [NVRTC-PR] Flowchart and file table (partial weight-gradient kernel, then a finalize kernel).
 *
 *   dy, x [rows, hidden] in_dtype; mu [rows] float32 (LayerNorm; NULL for RMSNorm);
 *   rsigma [rows] float32 (the forward's outputs); gamma [hidden] w_dtype.
 *   xhat = (x - mu) * rsigma (LayerNorm) or x * rsigma (RMSNorm); w = dy * g.
 *   dx = rsigma * (w - mean(w) - xhat * mean(w * xhat))  (LayerNorm),
 *   dx = rsigma * (w - xhat * mean(w * xhat))            (RMSNorm), stored in in_dtype.
 *   dgamma [hidden] w_dtype = sum over rows of dy * xhat; dbeta [hidden] w_dtype = sum of dy
 *   (LayerNorm only; NULL for RMSNorm). The row sums are reduced in a fixed order, so repeated
 *   calls give bitwise-identical results.
 */
int norm_bwd(void *stream, const void *dy, const void *x, const float *mu, const float *rsigma,
             const void *gamma, void *dx, void *dgamma, void *dbeta, void *workspace,
             size_t workspace_bytes, int64_t rows, int64_t hidden, int in_dtype, int w_dtype,
             int norm_type, int zero_centered_gamma, int cu_margin);

/*
 * norm_bwd_add -- fused RMSNorm backward plus residual gradient. [BwdAdd] Overview,
 * Description, I/O Contract: one kernel produces dx = rmsnorm_dx + residual_dy (summed in
 * float32, rounded once) and the weight gradient.
 *   residual_dy [rows, hidden] in_dtype; other arguments as norm_bwd with norm type RMSNorm.
 */
int norm_bwd_add(void *stream, const void *dy, const void *x, const void *residual_dy,
                 const float *rsigma, const void *gamma, void *dx, void *dgamma, void *workspace,
                 size_t workspace_bytes, int64_t rows, int64_t hidden, int in_dtype, int w_dtype,
                 int zero_centered_gamma, int cu_margin);

/*
 * norm_bwd_noalloc -- norm_bwd without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Arguments, results and errors are those of norm_bwd; the scratch memory the
 * backward's kernels need (the per-workgroup weight-gradient partials) is a static device array
 * of NORM_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the process ends.
 * The call allocates nothing. Shapes whose workspace query exceeds the array (LayerNorm rows of
 * more than about 16 K elements, RMSNorm of more than about 32 K) return NORM_ERR_UNSUPPORTED.
 * All calls on one GPU share its array: two calls that may overlap on one GPU (different
 * streams, or different threads without ordering) race and corrupt each other's gradients;
 * serialise them, or use norm_bwd with one workspace per stream.
 */
#define NORM_NOALLOC_SCRATCH_BYTES (32u << 20)
int norm_bwd_noalloc(void *stream, const void *dy, const void *x, const float *mu, const float *rsigma,
                     const void *gamma, void *dx, void *dgamma, void *dbeta, int64_t rows, int64_t hidden,
                     int in_dtype, int w_dtype, int norm_type, int zero_centered_gamma, int cu_margin);

/* Zero the synchronisation header of a new workspace (enqueues one small kernel on stream). */
int norm_workspace_init(void *stream, void *workspace, size_t workspace_bytes);

/*
 * Diagnostic, blocking: synchronises `stream`, copies the header's error word to *flags
 * (bit 0: a cross-workgroup wait exceeded its time limit; bit 1: header found corrupt) and
 * clears it. Not for the hot path.
 */
int norm_workspace_check(void *stream, void *workspace, uint32_t *flags);

/* The kernels a forward request goes to (norm_fwd_launch_shape). */
typedef enum {
  NORM_ROUTE_ROW = 0,               /* row kernel: one team of waves per row */
  NORM_ROUTE_ROW_TRANSPOSE = 1,     /* row kernel, then a byte transpose of its codes (delayed, both outputs) */
  NORM_ROUTE_STATS_TILES = 2,       /* statistics pass of the row kernel, then 128 x 128 tiles */
  NORM_ROUTE_BAND = 3,              /* band kernel: row tiles over S workgroups */
  NORM_ROUTE_SPLIT = 4,             /* split kernel: long rows over S workgroups */
  NORM_ROUTE_SINGLE_PASS_COLWISE = 5, /* single-pass columnwise kernel (RMSNorm FP8) */
  NORM_ROUTE_GENERAL = 6            /* general kernels (any hidden size) */
} norm_fwd_route_t;

/*
 * Planner query, host only (no GPU needed): the kernels norm_fwd chooses for these arguments
 * (those of norm_fwd_workspace_size that steer the plan). On return shape[0] = route
 * (norm_fwd_route_t); shape[1] = layout index (the row layout for routes ROW, ROW_TRANSPOSE and
 * STATS_TILES, the band layout for BAND, the split kernel's shape for SPLIT, else 0); shape[2] =
 * waves per row, shape[3] = 16-byte strips per lane and shape[4] = rows per workgroup of that row
 * layout (0 for other routes); shape[5] = S, the workgroups that share a row (BAND, SPLIT,
 * SINGLE_PASS_COLWISE; else 1). Tensors aligned only to their element size send a request to the
 * general kernels at launch, which this query does not see. [NVRTC-PR] Description and Flowchart
 * (the tuned kernel chosen per row length, the general kernel otherwise). For tests of the
 * planner's choices.
 */
int norm_fwd_launch_shape(int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int out_dtype, int norm_type,
                          int scaling, int qlayout, int cu_margin, int64_t shape[6]);

/*
 * Planner query, host only (no GPU needed): the launch shape norm_bwd / norm_bwd_add choose for
 * these arguments on a device with `cu_count` compute units, `cu_margin` of them left free,
 * when the backward row kernel fits `occupancy` workgroups per CU. On return shape[0] = layout
 * index (-1: the general kernels, the rest 0), shape[1] = waves per row team (W), shape[2] =
 * 16-byte strips per lane (KC), shape[3] = row teams per workgroup (T), shape[4] = workgroups in
 * the persistent grid (G). Workgroup b's team t visits rows b*T + t + j*G*T, j >= 0, for as long
 * as b*T + j*G*T < rows, and stores dx only for rows < rows. [NVRTC-PR] Flowchart (grid sizes
 * from occupancy and the SM margin). For tests that replay the kernel's row walk on the CPU.
 */
int norm_bwd_launch_shape(int64_t rows, int64_t hidden, int in_dtype, int w_dtype, int norm_type, int with_add,
                          int cu_count, int cu_margin, int occupancy, int64_t shape[5]);

/*
 * Tuning and test hook: sets one planner override for the whole process and returns the old
 * value in *previous (may be NULL). Each override starts from the environment variable of the
 * same name, read once when the library is first used; INT_MIN means "not set" (the planner's
 * default). Names: NORMFP8_ROW_CFG, NORMFP8_BAND_CFG, NORMFP8_BWD_CFG (force a kernel shape,
 * by its index in the library's shape tables), NORMFP8_FORCE_BAND (1: band kernel),
 * NORMFP8_COL_KERNEL (0: single-pass band kernel for columnwise output),
 * NORMFP8_DELAYED_TRANSPOSE (0: statistics + tile route for delayed scaling with both
 * outputs), NORMFP8_TRANSPOSE_TC / NORMFP8_TRANSPOSE_RL (byte-transpose tile shape),
 * NORMFP8_ROW_OCC (cap on row-kernel workgroups per CU), NORMFP8_ROW_BALANCE (0: plain
 * occupancy grid), NORMFP8_BAND_CLASSES (1: one ticket class), NORMFP8_SPLIT (0: no split
 * kernel for long rows; 1: split kernel for every row it covers), NORMFP8_COLX (0: two-pass
 * routes instead of the single-pass columnwise kernel), NORMFP8_SPLIT_SHAPE (0: the 16-wave
 * split shape, 16384-column slices; 1 / 2: the 8-wave shapes with 32768- / 16384-column slices,
 * 16-bit input).
 * Unknown names give
 * NORM_ERR_INVALID_ARG. Not for the hot path of an application: a change affects every later
 * call in the process.
 */
int norm_tuning_set(const char *name, int value, int *previous);

/* Message describing the last error returned on the calling thread ("" if none). */
const char *norm_last_error(void);

/* NORMFP8_ABI_VERSION of the built library. */
int norm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NORMFP8_H */
