"""fp64 CPU oracle of the fused per-state norm + FC step.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package smoke check and
by bench.py's cpu_baseline leg, never by the product path.  It shares no code
with the HIP library or its binding.
"""

from .fuse64 import (NORM_LN, NORM_NONE, NORM_RMS, decode_bf16, fold_apply, fold_prepare, fuse,
                     fuse_bits, normalize, round_bf16_rne, row_stats)
from .postnorm64 import norm_output, norm_output_bits
from .embedcat import embed_concat
from .verify64 import inverse_cdf, verify_accept

__all__ = [
    "NORM_NONE", "NORM_LN", "NORM_RMS", "decode_bf16", "row_stats", "normalize", "fuse", "fuse_bits",
    "fold_prepare", "fold_apply", "round_bf16_rne", "norm_output", "norm_output_bits", "embed_concat",
    "inverse_cdf", "verify_accept",
]
