"""LayerNorm / RMSNorm forward, FP8 epilogues and backward as plain float64 definitions.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in ``__graft_entry__``
and the CPU-baseline leg of ``bench.py`` may import anything under ``oracle/``;
the HIP library and its binding never do.  This is a slow, obviously-correct
reference: whole-array numpy expressions in float64, no blocking, no fusion.

Pages cited (by title and section):
  [XLA-Norm]  "Implementation: NVIDIA TransformerEngine JAX XLA Normalization"
  [BwdAdd]    "Implementation: NVIDIA TransformerEngine Ops Fused Backward Add RMSNorm"
  [NVRTC-PR]  "Migrate norms and softmax kernels to NVRTC" (TransformerEngine pull request)

The pages name the operations and their inputs/outputs but print no formula, so
each function below states the reading it implements:
  * LayerNorm statistics: mean and biased (population) variance of the row; the
    stability constant is added inside the square root: rsigma = 1/sqrt(var + eps).
  * RMSNorm statistics: mean of squares, no mean subtraction; rsigma = 1/sqrt(ms + eps).
  * "fp32 stats": the statistics are computed in float64 and each rounded once to
    binary32; the normalised values are then evaluated in float64 from those
    binary32 statistics (the values a fused kernel stores and reuses).
  * zero-centred gamma: the effective weight is 1 + gamma; beta is unchanged.
  * FP8 codes and MX exponents come from the unrounded float64 value: a delayed-
    scaling code is one nearest-even, saturating rounding of v * scale (the scale
    is a binary32 input); an MX block's exponent is taken from the float64 block
    maximum, and its codes are one rounding of v * 2**-X.  (A binary32 kernel
    reaches its codes through a chain of binary32 roundings; where that chain and
    this single rounding disagree the value lies on a rounding boundary, which the
    test-side checks verify element by element.)
  * Columnwise outputs are the same quantisation applied to the transposed
    matrix: layout [hidden, rows].
  * Backward: the exact gradient of sum(dy * y) with respect to x, gamma, beta,
    with mu and sigma treated as functions of x, evaluated at the saved stats.
"""
from __future__ import annotations

import numpy as np

from .formats import FORMATS, decode_storage, encode_storage, e8m0_exponent, fp8_quantize, to_f32

LAYERNORM = "layernorm"
RMSNORM = "rmsnorm"


# ----------------------------------------------------------------------------------------
# forward  ([XLA-Norm] Overview, Description, I/O Contract)
# ----------------------------------------------------------------------------------------

def row_stats(x, norm: str, eps: float, round_to_f32: bool = True):
    """Per-row statistics of x [rows, hidden] (float64).

    Returns (mu, rsigma); mu is None for RMSNorm ([XLA-Norm] I/O Contract: the mean
    output exists for LayerNorm only).  Two-pass in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[1]
    eps = float(eps)
    if norm == LAYERNORM:
        mu = x.sum(axis=1) / h
        var = ((x - mu[:, None]) ** 2).sum(axis=1) / h
        rs = 1.0 / np.sqrt(var + eps)
    elif norm == RMSNORM:
        mu = None
        ms = (x * x).sum(axis=1) / h
        rs = 1.0 / np.sqrt(ms + eps)
    else:
        raise ValueError(norm)
    if round_to_f32:
        rs = to_f32(rs)
        mu = to_f32(mu) if mu is not None else None
    return mu, rs


def effective_gamma(gamma, zero_centered_gamma: bool):
    """Weight applied to the normalised row: gamma, or 1 + gamma when zero-centred
    ([XLA-Norm] Signature / I/O Contract list zero_centered_gamma as an input)."""
    g = np.asarray(gamma, dtype=np.float64)
    return g + 1.0 if zero_centered_gamma else g


def normalized_values(x, mu, rs, g, beta, norm: str):
    """v = (x - mu) * rsigma * g + beta (LayerNorm) or x * rsigma * g (RMSNorm), float64."""
    x = np.asarray(x, dtype=np.float64)
    if norm == LAYERNORM:
        xhat = (x - mu[:, None]) * rs[:, None]
        return xhat * g[None, :] + np.asarray(beta, dtype=np.float64)[None, :]
    return x * rs[:, None] * g[None, :]


def forward(x, gamma, beta, norm: str, eps: float, zero_centered_gamma: bool = False,
            round_stats: bool = True):
    """Statistics and unrounded float64 outputs for float64 inputs.

    Returns dict(mu, rsigma, v).  mu is None for RMSNorm."""
    mu, rs = row_stats(x, norm, eps, round_to_f32=round_stats)
    g = effective_gamma(gamma, zero_centered_gamma)
    v = normalized_values(x, mu, rs, g, beta, norm)
    return {"mu": mu, "rsigma": rs, "v": v}


def plain_output(v, out_dtype: str):
    """No-scaling output: one nearest-even rounding of v to the output dtype
    ([XLA-Norm] Description: the no-scaling mode stores the high-precision result)."""
    return encode_storage(v, out_dtype)


# ----------------------------------------------------------------------------------------
# FP8 epilogues  ([XLA-Norm] Description: delayed tensor scaling, MXFP8 block scaling,
# rowwise with optional columnwise output; I/O Contract: scale and amax in, scale_inv
# and updated amax out)
# ----------------------------------------------------------------------------------------

def delayed_quantize(v, scale: float, fp8: str):
    """Per-tensor delayed scaling of a value matrix: codes = fp8(v * scale), one saturating
    nearest-even rounding of the float64 product of v and the binary32 scale."""
    return fp8_quantize(np.asarray(v, dtype=np.float64) * np.float64(np.float32(scale)), FORMATS[fp8])


def delayed_epilogue(v, scale: float, amax_in: float, fp8: str, colwise: bool):
    """All delayed-scaling outputs for one tensor.

    rowwise codes [rows, hidden]; colwise codes [hidden, rows] (quantisation of the
    transpose); updated amax = max(amax_in, max |v|) over the whole tensor; scale_inv
    = 1/scale in binary32 (also the colwise scale_inv)."""
    out = {"rowwise": delayed_quantize(v, scale, fp8)}
    if colwise:
        out["colwise"] = delayed_quantize(np.ascontiguousarray(np.asarray(v).T), scale, fp8)
    out["amax"] = max(float(amax_in), float(np.max(np.abs(v))) if np.size(v) else 0.0)
    out["scale_inv"] = np.float32(1.0) / np.float32(scale)
    return out


def mx_quantize_rows(v, fp8: str, block: int = 32, rule: str = "floor"):
    """MXFP8 along the last axis: blocks of ``block`` consecutive elements share one
    E8M0 scale (exponent rule ``rule``, see e8m0_exponent).  The last block of a row may be
    shorter.

    Returns (codes uint8 [r, c], scale bytes uint8 [r, ceil(c / block)])."""
    fmt = FORMATS[fp8]
    v = np.asarray(v, dtype=np.float64)
    r, c = v.shape
    nb = -(-c // block)
    codes = np.zeros((r, c), dtype=np.uint8)
    scales = np.zeros((r, nb), dtype=np.uint8)
    for b in range(nb):
        blk = v[:, b * block:(b + 1) * block]
        a = np.max(np.abs(blk), axis=1) if blk.shape[1] else np.zeros(r)
        x = e8m0_exponent(a, fp8, rule)
        scales[:, b] = (x + 127).astype(np.uint8)
        scaled = blk * np.ldexp(1.0, (-x)[:, None])       # exact power-of-two scaling
        codes[:, b * block:(b + 1) * block] = fp8_quantize(scaled, fmt)
    return codes, scales


def mx_epilogue(v, fp8: str, colwise: bool, block: int = 32, rule: str = "floor",
                col_layout: str = "transposed"):
    """MXFP8 outputs: rowwise data [rows, hidden] + scales [rows, ceil(hidden/32)];
    colwise data [hidden, rows] + scales [hidden, ceil(rows/32)] (blocks of 32
    consecutive rows of one column). col_layout "rowmajor" returns the same columnwise codes
    and scales in the rowwise orientation: data [rows, hidden], scales [ceil(rows/32), hidden]
    (a layout choice only; the arithmetic is the transposed case's)."""
    out = {}
    out["rowwise"], out["rowwise_scale"] = mx_quantize_rows(v, fp8, block, rule)
    if colwise:
        vt = np.ascontiguousarray(np.asarray(v).T)
        out["colwise"], out["colwise_scale"] = mx_quantize_rows(vt, fp8, block, rule)
        if col_layout == "rowmajor":
            out["colwise"] = np.ascontiguousarray(out["colwise"].T)
            out["colwise_scale"] = np.ascontiguousarray(out["colwise_scale"].T)
        elif col_layout != "transposed":
            raise ValueError(f"unknown columnwise layout {col_layout!r}")
    return out


# ----------------------------------------------------------------------------------------
# backward  ([XLA-Norm] Description: LayerNorm / RMSNorm backward; [NVRTC-PR] file table
# and flowchart: partial weight-gradient kernels followed by a finalize step;
# [BwdAdd] Overview, I/O Contract: RMSNorm backward plus the residual gradient)
# ----------------------------------------------------------------------------------------

def backward(dy, x, mu, rs, g, norm: str):
    """Gradients of L = sum(dy * y) at the saved statistics, float64.

    xhat = (x - mu) * rsigma (LayerNorm) or x * rsigma (RMSNorm); w = dy * g;
    dx = rsigma * (w - mean(w) - xhat * mean(w * xhat))   (LayerNorm)
    dx = rsigma * (w - xhat * mean(w * xhat))             (RMSNorm)
    dgamma = sum over rows of dy * xhat; dbeta = sum over rows of dy (LayerNorm).
    Returns dict(dx, dgamma, dbeta); dbeta is None for RMSNorm."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[1]
    rsc = np.asarray(rs, dtype=np.float64)[:, None]
    if norm == LAYERNORM:
        xhat = (x - np.asarray(mu, dtype=np.float64)[:, None]) * rsc
    else:
        xhat = x * rsc
    w = dy * np.asarray(g, dtype=np.float64)[None, :]
    c2 = (w * xhat).sum(axis=1, keepdims=True) / h
    if norm == LAYERNORM:
        c1 = w.sum(axis=1, keepdims=True) / h
        dx = rsc * (w - c1 - xhat * c2)
        dbeta = dy.sum(axis=0)
    else:
        dx = rsc * (w - xhat * c2)
        dbeta = None
    dgamma = (dy * xhat).sum(axis=0)
    return {"dx": dx, "dgamma": dgamma, "dbeta": dbeta}


def backward_add(dy, x, rs, g, residual_dy):
    """Fused RMSNorm backward + residual gradient: dx = rmsnorm_dx + residual_dy,
    summed in float64 before the single output rounding ([BwdAdd] I/O Contract)."""
    out = backward(dy, x, None, rs, g, RMSNORM)
    out["dx"] = out["dx"] + np.asarray(residual_dy, dtype=np.float64)
    return out


# ----------------------------------------------------------------------------------------
# convenience wrappers taking stored tensors (numpy, bf16 as uint16 bits)
# ----------------------------------------------------------------------------------------

def forward_stored(x, gamma, beta, *, norm, eps, in_dtype, w_dtype, zero_centered_gamma=False):
    """forward() on stored arrays; eps is used at its binary32 value (the API takes a float)."""
    xd = decode_storage(x, in_dtype)
    gd = decode_storage(gamma, w_dtype)
    bd = decode_storage(beta, w_dtype) if beta is not None else None
    return forward(xd, gd, bd, norm, float(np.float32(eps)), zero_centered_gamma)


def backward_stored(dy, x, mu, rs, gamma, *, norm, in_dtype, w_dtype, zero_centered_gamma=False,
                    residual_dy=None):
    """backward() / backward_add() on stored arrays with binary32 mu / rsigma."""
    dyd = decode_storage(dy, in_dtype)
    xd = decode_storage(x, in_dtype)
    g = effective_gamma(decode_storage(gamma, w_dtype), zero_centered_gamma)
    mu64 = None if mu is None else np.asarray(mu, dtype=np.float32).astype(np.float64)
    rs64 = np.asarray(rs, dtype=np.float32).astype(np.float64)
    if residual_dy is not None:
        assert norm == RMSNORM
        return backward_add(dyd, xd, rs64, g, decode_storage(residual_dy, in_dtype))
    return backward(dyd, xd, mu64, rs64, g, norm)
