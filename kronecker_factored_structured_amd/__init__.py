"""Kronecker-factored structured layers on AMD MI355X (gfx950).

The compute lives in libkron.so (HIP kernels behind a C ABI, include/kron.h); this
package is its Python binding.  Build the library with
`python -m kronecker_factored_structured_amd.build`.
"""
from . import _lib
from .api import (kron_adam_l1_step, kron_head_ce, kron_l1_penalty, kron_l1_penalty_grad, kron_linear_bwd,
                  kron_linear_bwd_bf16, kron_linear_bwd_noalloc, kron_linear_bwd_bf16_workspace_bytes,
                  kron_linear_bwd_workspace_bytes, kron_linear_zcache_bytes, new_zcache, kron_linear_fwd, kron_linear_fwd_bf16, kron_relu_bwd, kron_van_loan, ks_chain, ks_matmul,
                  ks_matmul_bwd, ks_matmul_bwd_workspace_bytes, ks_matmul_out, layer_shape)
from .layers import KronLinear, KronMLPStep, KSLinear

__all__ = [
    "kron_linear_fwd", "kron_linear_bwd", "kron_linear_bwd_workspace_bytes", "ks_matmul",
    "kron_adam_l1_step", "kron_head_ce", "layer_shape", "KronLinear", "KSLinear", "KronMLPStep", "_lib",
    "kron_linear_fwd_bf16", "kron_linear_bwd_bf16", "kron_linear_bwd_bf16_workspace_bytes", "ks_matmul_out",
    "ks_matmul_bwd", "ks_matmul_bwd_workspace_bytes", "ks_chain", "kron_van_loan", "kron_relu_bwd",
    "kron_l1_penalty", "kron_l1_penalty_grad", "kron_linear_bwd_noalloc", "kron_linear_zcache_bytes", "new_zcache",
]
