"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds only input recipes: shapes, dtypes, seeds and value
distributions.  It contains none of the normalisation or quantisation
arithmetic, so that the CPU oracle and the HIP library can both be fed from it
without sharing any of the method.

Recipe (applies to every generator here):
  * one ``torch.Generator('cpu')`` per tensor, seeded ``base + role`` where the
    role offsets are x=0, gamma=1, beta=2, dy=3, residual_dy=4, outlier mask=5,
    prior batch=6;
  * ``torch.randn`` in float32, then the affine map of the recipe
    (``N(m, s)`` means mean m and standard deviation s), then one round-to-
    nearest-even cast to the tensor's storage dtype;
  * outliers (the delayed-scaling workload): a Bernoulli(p) mask drawn with
    ``torch.rand < p`` from its own generator; masked elements are multiplied
    by the outlier factor before the cast.

The six named workloads follow the workload list of the benchmark: an fp32
RMSNorm at 256 x 1024, a bf16 LayerNorm at 16384 x 4096, a bf16 RMSNorm with
delayed per-tensor E4M3 output at 32768 x 8192, a bf16 RMSNorm with MXFP8 output
at 16384 x 12288, a bf16 LayerNorm with very long rows at 1024 x 65536, and the
fused backward-add RMSNorm at 32768 x 8192.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

ROLE_X, ROLE_GAMMA, ROLE_BETA, ROLE_DY, ROLE_RES, ROLE_MASK, ROLE_PRIOR = range(7)

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Dist:
    """Normal distribution N(mean, std), optional outliers (probability, factor)."""
    mean: float = 0.0
    std: float = 1.0
    outlier_p: float = 0.0
    outlier_scale: float = 1.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    norm: str                 # "layernorm" | "rmsnorm"
    rows: int
    hidden: int
    in_dtype: str             # storage dtype of x, y, dy, dx, residual_dy
    w_dtype: str              # storage dtype of gamma, beta, dgamma, dbeta
    x: Dist
    gamma: Dist
    beta: Optional[Dist]
    dy: Optional[Dist]
    residual: Optional[Dist]
    zero_centered_gamma: bool
    scaling: str              # "none" | "delayed" | "mxfp8"
    fp8: str                  # "e4m3" | "e5m2" (ignored when scaling == "none")
    colwise: bool
    passes: tuple             # subset of ("fwd", "bwd", "bwd_add")
    seed_base: int
    eps: float = 1e-5

    def scaled(self, rows: Optional[int] = None, hidden: Optional[int] = None,
               name: Optional[str] = None) -> "Workload":
        """Same recipe at another shape (used for small parity cases)."""
        return dataclasses.replace(self, rows=rows if rows is not None else self.rows,
                                   hidden=hidden if hidden is not None else self.hidden,
                                   name=name or self.name)


WORKLOADS: Dict[str, Workload] = {
    "rms_f32_256x1024": Workload(
        "rms_f32_256x1024", "rmsnorm", 256, 1024, "f32", "f32",
        x=Dist(0.0, 1.0), gamma=Dist(1.0, 0.1), beta=None, dy=Dist(0.0, 1.0), residual=None,
        zero_centered_gamma=False, scaling="none", fp8="e4m3", colwise=False,
        passes=("fwd", "bwd"), seed_base=1000),
    "ln_bf16_16384x4096": Workload(
        "ln_bf16_16384x4096", "layernorm", 16384, 4096, "bf16", "f32",
        x=Dist(0.5, 3.0), gamma=Dist(1.0, 0.1), beta=Dist(0.0, 0.1), dy=Dist(0.0, 1.0),
        residual=None, zero_centered_gamma=False, scaling="none", fp8="e4m3", colwise=False,
        passes=("fwd", "bwd"), seed_base=2000),
    "rms_bf16_32768x8192_delayed_e4m3": Workload(
        "rms_bf16_32768x8192_delayed_e4m3", "rmsnorm", 32768, 8192, "bf16", "f32",
        x=Dist(0.0, 1.0, outlier_p=1e-3, outlier_scale=20.0), gamma=Dist(1.0, 0.1), beta=None,
        dy=None, residual=None, zero_centered_gamma=False, scaling="delayed", fp8="e4m3",
        colwise=True, passes=("fwd",), seed_base=3000),
    "rms_bf16_16384x12288_mxfp8_e4m3": Workload(
        "rms_bf16_16384x12288_mxfp8_e4m3", "rmsnorm", 16384, 12288, "bf16", "f32",
        x=Dist(0.0, 1.0), gamma=Dist(0.0, 0.05), beta=None, dy=None, residual=None,
        zero_centered_gamma=True, scaling="mxfp8", fp8="e4m3", colwise=True,
        passes=("fwd",), seed_base=4000),
    "ln_bf16_1024x65536": Workload(
        "ln_bf16_1024x65536", "layernorm", 1024, 65536, "bf16", "f32",
        x=Dist(0.5, 3.0), gamma=Dist(1.0, 0.1), beta=Dist(0.0, 0.1), dy=None, residual=None,
        zero_centered_gamma=False, scaling="none", fp8="e4m3", colwise=False,
        passes=("fwd",), seed_base=4500),
    "rms_bf16_32768x8192_bwd_add": Workload(
        "rms_bf16_32768x8192_bwd_add", "rmsnorm", 32768, 8192, "bf16", "f32",
        x=Dist(0.0, 1.0), gamma=Dist(1.0, 0.1), beta=None, dy=Dist(0.0, 1.0),
        residual=Dist(0.0, 0.5), zero_centered_gamma=False, scaling="none", fp8="e4m3",
        colwise=False, passes=("bwd_add",), seed_base=5000),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator("cpu")
    g.manual_seed(int(seed))
    return g


def draw(shape, dist: Dist, dtype: str, seed: int, mask_seed: Optional[int] = None) -> torch.Tensor:
    """One seeded tensor of the recipe: randn -> affine -> optional outliers -> cast."""
    t = torch.randn(*shape, generator=_gen(seed), dtype=torch.float32)
    t.mul_(dist.std).add_(dist.mean)
    if dist.outlier_p > 0.0:
        assert mask_seed is not None
        m = torch.rand(*shape, generator=_gen(mask_seed), dtype=torch.float32) < dist.outlier_p
        t[m] *= dist.outlier_scale
    return t.to(TORCH_DTYPES[dtype])


def make_inputs(w: Workload, prior: bool = False) -> Dict[str, torch.Tensor]:
    """Host (CPU) tensors for one batch of the workload.

    ``prior=True`` draws the previous step's batch of x (used to derive the
    delayed-scaling factor); every other tensor is identical.
    """
    b = w.seed_base
    shape = (w.rows, w.hidden)
    xs = b + (ROLE_PRIOR if prior else ROLE_X)
    out = {"x": draw(shape, w.x, w.in_dtype, xs, mask_seed=xs + 100 + ROLE_MASK)}
    out["gamma"] = draw((w.hidden,), w.gamma, w.w_dtype, b + ROLE_GAMMA)
    if w.norm == "layernorm":
        out["beta"] = draw((w.hidden,), w.beta or Dist(0.0, 0.1), w.w_dtype, b + ROLE_BETA)
    if w.dy is not None:
        out["dy"] = draw(shape, w.dy, w.in_dtype, b + ROLE_DY)
    if w.residual is not None:
        out["residual_dy"] = draw(shape, w.residual, w.in_dtype, b + ROLE_RES)
    return out


def small_case(norm: str, rows: int, hidden: int, in_dtype: str = "bf16", w_dtype: str = "f32",
               seed: int = 7, zero_centered_gamma: bool = False, x_mean: float = 0.5,
               x_std: float = 3.0) -> Dict[str, torch.Tensor]:
    """Generic seeded case for parity tests at arbitrary (small) shapes."""
    shape = (rows, hidden)
    gd = Dist(0.0, 0.05) if zero_centered_gamma else Dist(1.0, 0.1)
    out = {"x": draw(shape, Dist(x_mean, x_std), in_dtype, seed * 10 + ROLE_X),
           "gamma": draw((hidden,), gd, w_dtype, seed * 10 + ROLE_GAMMA),
           "dy": draw(shape, Dist(0.0, 1.0), in_dtype, seed * 10 + ROLE_DY),
           "residual_dy": draw(shape, Dist(0.0, 0.5), in_dtype, seed * 10 + ROLE_RES)}
    if norm == "layernorm":
        out["beta"] = draw((hidden,), Dist(0.0, 0.1), w_dtype, seed * 10 + ROLE_BETA)
    return out


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Host tensor -> numpy array holding the exact stored values.

    float32 and float16 come back as their own numpy dtypes; bfloat16 (which numpy
    lacks) comes back as its raw uint16 bit patterns.
    """
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
