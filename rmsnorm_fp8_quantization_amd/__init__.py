"""Fused LayerNorm / RMSNorm + FP8 quantisation for AMD MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI of ``include/normfp8.h``
(``libnormfp8.so``, built in-tree by ``python -m rmsnorm_fp8_quantization_amd.build``).
This package is its thin Python binding:

* ``_lib`` -- ctypes entry points with the C names (``norm_fwd``, ``norm_bwd``, ...);
* ``ops``  -- torch-tensor wrappers ``fwd``, ``bwd``, ``bwd_add``;
* ``autograd`` -- differentiable ``layer_norm``, ``rms_norm`` and ``rms_norm_residual`` (the
  fused backward-add for a norm whose input also feeds a residual branch).

The library is loaded on first use; if it has not been built, that first use raises.
"""
from . import _lib, autograd
from .ops import (bwd, bwd_add, bwd_workspace_size, fwd, fwd_workspace_size, prepare_bwd,
                  prepare_bwd_add, prepare_fwd, workspace_check)

__all__ = ["fwd", "bwd", "bwd_add", "prepare_fwd", "prepare_bwd", "prepare_bwd_add",
           "fwd_workspace_size", "bwd_workspace_size", "workspace_check", "_lib", "autograd"]
