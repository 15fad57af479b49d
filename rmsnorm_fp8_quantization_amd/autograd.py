"""torch.autograd functions over the fused kernels.

Pages cited (by title and section): [XLA-Norm] "Implementation: NVIDIA TransformerEngine JAX
XLA Normalization" (Usage: the forward and backward are registered as one differentiable
operation); [BwdAdd] "Implementation: NVIDIA TransformerEngine Ops Fused Backward Add RMSNorm"
(Overview, Description: when the normalised tensor also feeds a residual branch, the RMSNorm
backward adds that branch's gradient into grad_input inside the same kernel).

* ``layer_norm(x, gamma, beta, eps, zero_centered_gamma)`` and
  ``rms_norm(x, gamma, eps, zero_centered_gamma)``: y in x's dtype; gradients for x, gamma and
  beta come from ``norm_bwd``.
* ``rms_norm_residual(x, gamma, eps, zero_centered_gamma)`` returns ``(y, x_res)``, where
  ``x_res`` is x itself for the residual branch. In the backward, the gradient arriving at
  ``x_res`` is added to the norm's dx by ``norm_bwd_add`` (one kernel) instead of by a separate
  autograd accumulation.

Leading dimensions are flattened: x is [..., hidden]. Every computation runs in the HIP
kernels; this module only reshapes and routes tensors.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import ops


def _rows(t: torch.Tensor) -> torch.Tensor:
    return t.reshape(-1, t.shape[-1]).contiguous()


class _Norm(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, gamma, beta, norm: str, eps: float, zero_centered_gamma: bool):
        x2 = _rows(x)
        out = ops.fwd(x2, gamma, beta, norm=norm, eps=eps, zero_centered_gamma=zero_centered_gamma)
        ctx.save_for_backward(x2, gamma, out["mu"], out["rsigma"])
        ctx.norm = norm
        ctx.zero_centered_gamma = zero_centered_gamma
        ctx.has_beta = beta is not None
        ctx.shape = x.shape
        return out["y"].view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, gamma, mu, rs = ctx.saved_tensors
        g = ops.bwd(_rows(dy), x2, mu, rs, gamma, norm=ctx.norm,
                    zero_centered_gamma=ctx.zero_centered_gamma)
        db = g["dbeta"] if ctx.has_beta else None
        return g["dx"].view(ctx.shape), g["dgamma"], db, None, None, None


class _RMSNormResidual(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, gamma, eps: float, zero_centered_gamma: bool):
        x2 = _rows(x)
        out = ops.fwd(x2, gamma, None, norm="rmsnorm", eps=eps, zero_centered_gamma=zero_centered_gamma)
        ctx.save_for_backward(x2, gamma, out["rsigma"])
        ctx.zero_centered_gamma = zero_centered_gamma
        ctx.shape = x.shape
        return out["y"].view(x.shape), x

    @staticmethod
    def backward(ctx, dy, dres):
        x2, gamma, rs = ctx.saved_tensors
        zc = ctx.zero_centered_gamma
        if dy is None:
            dy = torch.zeros(ctx.shape, dtype=x2.dtype, device=x2.device)
        if dres is None:
            g = ops.bwd(_rows(dy), x2, None, rs, gamma, norm="rmsnorm", zero_centered_gamma=zc)
        else:
            g = ops.bwd_add(_rows(dy), x2, _rows(dres.to(x2.dtype)), rs, gamma, zero_centered_gamma=zc)
        return g["dx"].view(ctx.shape), g["dgamma"], None, None


def layer_norm(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float = 1e-5,
               zero_centered_gamma: bool = False) -> torch.Tensor:
    """Differentiable LayerNorm over the last dimension (y in x's dtype)."""
    return _Norm.apply(x, gamma, beta, "layernorm", eps, zero_centered_gamma)


def rms_norm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5,
             zero_centered_gamma: bool = False) -> torch.Tensor:
    """Differentiable RMSNorm over the last dimension (y in x's dtype)."""
    return _Norm.apply(x, gamma, None, "rmsnorm", eps, zero_centered_gamma)


def rms_norm_residual(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5,
                      zero_centered_gamma: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """(RMSNorm(x), x): use the second output for the residual branch; its gradient is added to
    dx inside the fused backward-add kernel."""
    return _RMSNormResidual.apply(x, gamma, eps, zero_centered_gamma)


__all__ = ["layer_norm", "rms_norm", "rms_norm_residual"]
