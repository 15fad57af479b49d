"""Torch-facing wrappers of the C ABI: allocate outputs with torch, pass device pointers
and the current HIP stream, call ``norm_fwd`` / ``norm_bwd`` / ``norm_bwd_add``.

Pages cited (by title and section): [XLA-Norm] "Implementation: NVIDIA TransformerEngine JAX
XLA Normalization" (Description, Signature, I/O Contract: the forward's inputs and outputs);
[BwdAdd] "Implementation: NVIDIA TransformerEngine Ops Fused Backward Add RMSNorm" (I/O
Contract: grad_input = RMSNorm backward + residual gradient, and the weight gradient).

Nothing here computes: every element of every output is produced by the HIP kernels.
``prepare_fwd`` / ``prepare_bwd`` / ``prepare_bwd_add`` allocate the outputs and pack the
foreign-call arguments once, returning a callable that enqueues the kernels again on the
same buffers with a single foreign call (for timing loops and graph capture).
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Tuple

import torch

from . import _lib as L

_DT = {torch.float32: L.NORM_F32, torch.float16: L.NORM_F16, torch.bfloat16: L.NORM_BF16}
_FP8 = {"e4m3": L.NORM_FP8_E4M3, "e5m2": L.NORM_FP8_E5M2}
_NORM = {"layernorm": L.NORM_LAYERNORM, "rmsnorm": L.NORM_RMSNORM}
_SCALING = {"none": L.NORM_SCALING_NONE, "delayed": L.NORM_SCALING_DELAYED_TENSOR,
            "mxfp8": L.NORM_SCALING_MXFP8_1D32, "mxfp8_ceil": L.NORM_SCALING_MXFP8_1D32_CEIL}
_LAYOUT = {"rowwise": L.NORM_Q_ROWWISE, "colwise": L.NORM_Q_COLWISE,
           "rowwise_colwise": L.NORM_Q_ROWWISE_COLWISE,
           # columnwise output kept in the [rows, hidden] layout
           "colwise_rowmajor": L.NORM_Q_COLWISE | L.NORM_Q_COLWISE_ROWMAJOR,
           "rowwise_colwise_rowmajor": L.NORM_Q_ROWWISE_COLWISE | L.NORM_Q_COLWISE_ROWMAJOR}

_ws_cache: Dict[tuple, torch.Tensor] = {}
# workspaces replaced by larger ones: kept, never freed, because a prepared call or a captured
# graph may still point at them (sizes at least double, so few are kept)
_ws_retired: Dict[tuple, list] = {}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Prepared:
    """One entry point with its packed arguments; calling it enqueues the kernels again."""

    def __init__(self, name: str, args: tuple, keep: tuple):
        self.name = name
        self.fn = getattr(L.load(), name)
        self.args = args
        self._keep = keep       # tensors whose memory the arguments point to

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != L.NORM_OK:
            raise L.NormError(self.name, rc, L.load().norm_last_error().decode())


def workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-initialised workspace for the current stream of ``device`` (grown on demand).

    The library keeps the workspace's synchronisation header zeroed between calls, so a
    buffer is zero-filled only when first allocated. A buffer outgrown by a larger request is
    not freed: calls prepared earlier (``prepare_*``) and graphs captured from them keep
    pointing at it, so it stays referenced for the life of the process. Each replacement at
    least doubles the size."""
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(dev).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(nbytes, L.NORM_WS_HEADER_BYTES)
        if ws is not None:
            size = max(size, 2 * ws.numel())
            _ws_retired.setdefault(key, []).append(ws)
        ws = torch.zeros(size, dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


def _round_up(a: int, b: int) -> int:
    return (a + b - 1) // b * b


def fwd_workspace_size(rows, hidden, in_dtype, w_dtype, out_code, norm, scaling, layout,
                       zero_centered_gamma=False, eps=1e-5, cu_margin=0, training=True) -> int:
    """layout: a layout name, or the ABI's qlayout code (modifiers included)."""
    n = ctypes.c_size_t(0)
    code = _LAYOUT[layout] if isinstance(layout, str) else int(layout)
    L.call("norm_fwd_workspace_size", rows, hidden, _DT[in_dtype], _DT[w_dtype], out_code,
           _NORM[norm], _SCALING[scaling], code, int(zero_centered_gamma), eps,
           cu_margin, int(training), ctypes.byref(n))
    return n.value


def bwd_workspace_size(rows, hidden, in_dtype, w_dtype, norm, with_add=False,
                       zero_centered_gamma=False, eps=1e-5, cu_margin=0) -> int:
    n = ctypes.c_size_t(0)
    L.call("norm_bwd_workspace_size", rows, hidden, _DT[in_dtype], _DT[w_dtype], _NORM[norm],
           int(zero_centered_gamma), eps, cu_margin, int(with_add), ctypes.byref(n))
    return n.value


def prepare_fwd(x: torch.Tensor, gamma: torch.Tensor, beta: Optional[torch.Tensor] = None, *,
                norm: str = "rmsnorm", eps: float = 1e-5, zero_centered_gamma: bool = False,
                scaling: str = "none", out_dtype: Optional[torch.dtype] = None, fp8: str = "e4m3",
                scale: Optional[torch.Tensor] = None, amax: Optional[torch.Tensor] = None,
                layout: str = "rowwise", cu_margin: int = 0, training: bool = True,
                amax_inplace: bool = False, scales_padded: bool = False) -> Tuple[Dict[str, torch.Tensor], Prepared]:
    """Allocate the forward's outputs and pack a ``norm_fwd`` call (see ``fwd``)."""
    _check(x, "x")
    _check(gamma, "gamma")
    if beta is not None:
        _check(beta, "beta")
    if x.dim() != 2:
        raise ValueError("x must be [rows, hidden]")
    rows, hidden = x.shape
    dev = x.device
    rowwise = layout in ("rowwise", "rowwise_colwise", "rowwise_colwise_rowmajor")
    colwise = layout != "rowwise"
    col_rowmajor = layout.endswith("_rowmajor")
    if scaling == "none":
        odt = out_dtype or x.dtype
        out_code = _DT[odt]
        y = torch.empty(rows, hidden, dtype=odt, device=dev)
    else:
        out_code = _FP8[fp8]
        y = torch.empty(rows, hidden, dtype=torch.uint8, device=dev) if rowwise else None
    y_col = (torch.empty(*((rows, hidden) if col_rowmajor else (hidden, rows)), dtype=torch.uint8, device=dev)
             if colwise else None)
    mu = torch.empty(rows, dtype=torch.float32, device=dev) if norm == "layernorm" else None
    rs = torch.empty(rows, dtype=torch.float32, device=dev)
    si = csi = upd = None
    if scaling == "delayed":
        if scale is None or amax is None:
            raise ValueError("delayed scaling needs scale and amax tensors")
        si = torch.empty(1, dtype=torch.float32, device=dev) if rowwise else None
        csi = torch.empty(1, dtype=torch.float32, device=dev) if colwise else None
        upd = amax if amax_inplace else torch.empty(1, dtype=torch.float32, device=dev)
    elif scaling in ("mxfp8", "mxfp8_ceil"):
        # E8M0 grids; padded: the block-count dimension to a multiple of 4, the other to 128
        def grid(a, blocks):
            return (_round_up(a, 128), _round_up(blocks, 4)) if scales_padded else (a, blocks)
        si = torch.empty(*grid(rows, (hidden + 31) // 32), dtype=torch.uint8, device=dev) if rowwise else None
        if col_rowmajor:
            csi_shape = grid(hidden, (rows + 31) // 32)[::-1]
        else:
            csi_shape = grid(hidden, (rows + 31) // 32)
        csi = torch.empty(*csi_shape, dtype=torch.uint8, device=dev) if colwise else None
    if scales_padded and scaling not in ("mxfp8", "mxfp8_ceil"):
        raise ValueError("scales_padded applies to MXFP8 scaling only")
    lcode = _LAYOUT[layout] | (L.NORM_Q_SCALES_PADDED if scales_padded else 0)
    nbytes = fwd_workspace_size(rows, hidden, x.dtype, gamma.dtype, out_code, norm, scaling, lcode,
                                zero_centered_gamma, eps, cu_margin, training)
    ws = workspace(nbytes, dev) if nbytes else None
    args = (_stream(dev), _ptr(x), _ptr(gamma), _ptr(beta), _ptr(scale), _ptr(amax), _ptr(y), _ptr(y_col),
            _ptr(mu), _ptr(rs), _ptr(si), _ptr(csi), _ptr(upd), _ptr(ws), ws.numel() if ws is not None else 0,
            rows, hidden, _DT[x.dtype], _DT[gamma.dtype], out_code, _NORM[norm], _SCALING[scaling],
            lcode, int(zero_centered_gamma), eps, cu_margin)
    out = {"y": y, "y_colwise": y_col, "mu": mu, "rsigma": rs, "scale_inv": si, "colwise_scale_inv": csi,
           "amax": upd}
    keep = (x, gamma, beta, scale, amax, y, y_col, mu, rs, si, csi, upd, ws)
    return out, Prepared("norm_fwd", args, keep)


def fwd(x: torch.Tensor, gamma: torch.Tensor, beta: Optional[torch.Tensor] = None,
        **kw) -> Dict[str, torch.Tensor]:
    """LayerNorm / RMSNorm forward with an optional FP8 epilogue (one kernel launch; two for a
    columnwise output: row statistics, then 128 x 128 tiles; or, for delayed scaling with both
    outputs, the rowwise codes, then their transpose).

    x: [rows, hidden] (f32/f16/bf16); gamma, beta: [hidden]. Keywords: norm ("layernorm" |
    "rmsnorm"), eps, zero_centered_gamma, scaling ("none" | "delayed" | "mxfp8" | "mxfp8_ceil": MXFP8 with the round-up exponent
    rule, no saturation), out_dtype
    (scaling "none"), fp8 ("e4m3" | "e5m2"), scale / amax (float32[1] GPU tensors, delayed
    scaling), layout ("rowwise" | "colwise" | "rowwise_colwise", or "colwise_rowmajor" /
    "rowwise_colwise_rowmajor" for a columnwise output kept in the [rows, hidden] layout, with MXFP8
    columnwise scales [ceil(rows/32), hidden]), cu_margin, amax_inplace, scales_padded (MXFP8:
    E8M0 grids with the block-count dimension rounded up to a multiple of 4 and the other to a
    multiple of 128; only the logical region is written).
    Returns ``y`` (rowwise output: out_dtype, or uint8 FP8 codes), ``y_colwise`` ([hidden, rows]
    uint8 codes), ``mu`` (LayerNorm), ``rsigma``, ``scale_inv`` / ``colwise_scale_inv``
    (float32[1] for delayed scaling, uint8 E8M0 grids for MXFP8) and ``amax`` (updated amax)."""
    out, call = prepare_fwd(x, gamma, beta, **kw)
    with torch.cuda.device(x.device):
        call()
    return out


def prepare_bwd(dy: torch.Tensor, x: torch.Tensor, mu: Optional[torch.Tensor], rsigma: torch.Tensor,
                gamma: torch.Tensor, *, norm: str = "rmsnorm", zero_centered_gamma: bool = False,
                cu_margin: int = 0) -> Tuple[Dict[str, torch.Tensor], Prepared]:
    for t, n in ((dy, "dy"), (x, "x"), (rsigma, "rsigma"), (gamma, "gamma")):
        _check(t, n)
    rows, hidden = x.shape
    dev = x.device
    dx = torch.empty_like(x)
    dg = torch.empty_like(gamma)
    db = torch.empty_like(gamma) if norm == "layernorm" else None
    nbytes = bwd_workspace_size(rows, hidden, x.dtype, gamma.dtype, norm, False, zero_centered_gamma,
                                1e-5, cu_margin)
    ws = workspace(nbytes, dev)
    args = (_stream(dev), _ptr(dy), _ptr(x), _ptr(mu), _ptr(rsigma), _ptr(gamma), _ptr(dx), _ptr(dg),
            _ptr(db), _ptr(ws), ws.numel(), rows, hidden, _DT[x.dtype], _DT[gamma.dtype], _NORM[norm],
            int(zero_centered_gamma), cu_margin)
    return ({"dx": dx, "dgamma": dg, "dbeta": db},
            Prepared("norm_bwd", args, (dy, x, mu, rsigma, gamma, dx, dg, db, ws)))


def bwd(dy, x, mu, rsigma, gamma, **kw) -> Dict[str, torch.Tensor]:
    """LayerNorm / RMSNorm backward: dx (x's dtype), dgamma and dbeta (gamma's dtype)."""
    out, call = prepare_bwd(dy, x, mu, rsigma, gamma, **kw)
    with torch.cuda.device(x.device):
        call()
    return out


def prepare_bwd_add(dy: torch.Tensor, x: torch.Tensor, residual_dy: torch.Tensor, rsigma: torch.Tensor,
                    gamma: torch.Tensor, *, zero_centered_gamma: bool = False,
                    cu_margin: int = 0) -> Tuple[Dict[str, torch.Tensor], Prepared]:
    for t, n in ((dy, "dy"), (x, "x"), (residual_dy, "residual_dy"), (rsigma, "rsigma"),
                 (gamma, "gamma")):
        _check(t, n)
    rows, hidden = x.shape
    dev = x.device
    dx = torch.empty_like(x)
    dg = torch.empty_like(gamma)
    nbytes = bwd_workspace_size(rows, hidden, x.dtype, gamma.dtype, "rmsnorm", True,
                                zero_centered_gamma, 1e-5, cu_margin)
    ws = workspace(nbytes, dev)
    args = (_stream(dev), _ptr(dy), _ptr(x), _ptr(residual_dy), _ptr(rsigma), _ptr(gamma), _ptr(dx),
            _ptr(dg), _ptr(ws), ws.numel(), rows, hidden, _DT[x.dtype], _DT[gamma.dtype],
            int(zero_centered_gamma), cu_margin)
    return ({"dx": dx, "dgamma": dg},
            Prepared("norm_bwd_add", args, (dy, x, residual_dy, rsigma, gamma, dx, dg, ws)))


def bwd_add(dy, x, residual_dy, rsigma, gamma, **kw) -> Dict[str, torch.Tensor]:
    """Fused RMSNorm backward + residual gradient: dx = rmsnorm_dx + residual_dy, and dgamma."""
    out, call = prepare_bwd_add(dy, x, residual_dy, rsigma, gamma, **kw)
    with torch.cuda.device(x.device):
        call()
    return out


def workspace_check(device=None) -> int:
    """Blocking diagnostic: error flags of the current stream's workspace (0 = clean)."""
    dev = torch.device(device or "cuda")
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(dev).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None:
        return 0
    flags = ctypes.c_uint32(0)
    L.call("norm_workspace_check", _stream(dev), _ptr(ws), ctypes.byref(flags))
    return flags.value
