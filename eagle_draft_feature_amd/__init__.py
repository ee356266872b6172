"""EAGLE-3.1 normalized multi-layer feature fusion on MI355X (gfx950).

    out = [norm(h_low) | norm(h_mid) | norm(h_high)] @ W + bias

with a per-state LayerNorm (gamma_s, beta_s) or RMSNorm (gamma_s), or no norm
(EAGLE-3).  Every step runs in the HIP kernels of libeagle31.so; this package
only marshals torch tensors (device memory and the current stream) into the
C ABI declared in include/eagle31.h.
"""

from __future__ import annotations

from ._capi import (NORM_LAYERNORM, NORM_NONE, NORM_RMSNORM, Eagle31Error, LIB_PATH, lib)
from .ops import (debug_fail_workspace_zero, debug_stats_recompute, embed_concat, fold_prepare, fuse, fuse_folded,
                  fuse_folded_noalloc, fuse_folded_rows, fuse_rows, fuse_ws, noalloc_scratch_bytes, norm_kind, norm_output, release, row_stats,
                  verify_accept, verify_chunking, workspace_init, workspace_size)

__all__ = [
    "debug_fail_workspace_zero", "fuse_folded_noalloc", "noalloc_scratch_bytes", "NORM_NONE", "NORM_LAYERNORM", "NORM_RMSNORM", "Eagle31Error", "LIB_PATH", "lib", "fuse", "fuse_ws",
    "fold_prepare", "fuse_folded", "fuse_rows", "fuse_folded_rows", "row_stats", "workspace_size", "workspace_init", "release", "norm_kind", "norm_output", "embed_concat", "debug_stats_recompute", "verify_accept", "verify_chunking",
]
