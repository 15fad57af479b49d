"""CPU oracle for the fused LayerNorm/RMSNorm + FP8 path (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, call or execute anything in this
package.  The product path (the HIP library under
``rmsnorm_fp8_quantization_amd/`` and its Python binding) must never import it,
and this package imports nothing from the product path: the two share no
kernels, headers, helpers, tables or constants.  The only module both sides
are fed from is ``workloads`` (seeded inputs, no arithmetic of the method).

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, brute force, finite differences and library routines (torch float64
layer_norm / rms_norm / autograd, torch FP8 casts inside the finite range).
Readings that nothing on the pages can arbitrate -- and that are therefore
"parity unpinned" against the pages themselves -- are: the FP8 saturation rule,
the E8M0 floor rule, the transposed [hidden, rows] columnwise layout, and the
max-accumulation of the amax input.
"""
from .formats import (BF16, E4M3, E5M2, FORMATS, FP16, FP32, MX_EMAX, decode_storage,
                      e8m0_exponent, encode_storage, floor_log2, fp8_decode, fp8_encode,
                      fp8_quantize, round_nearest_even, to_f32)
from .norm import (LAYERNORM, RMSNORM, backward, backward_add, backward_stored,
                   delayed_epilogue, delayed_quantize, effective_gamma, forward,
                   forward_stored, mx_epilogue, mx_quantize_rows, normalized_values,
                   plain_output, row_stats)
