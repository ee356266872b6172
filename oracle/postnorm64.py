"""fp64 CPU oracle of the post-norm hidden-state feedback.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the bench's
cpu_baseline leg may import this module.  It shares no code with the device
path.

What it computes (vLLM EAGLE 3.1 release post,
devlery.com/blog/vllm-eagle31-attention-drift, section "EAGLE 3.1이 바꾼 것은
작지만 낮은 계층입니다": the second of EAGLE 3.1's two changes is that the
drafter feeds its post-norm hidden state to the next decoding step; section
"vLLM main에 들어갔다는 것이 뉴스입니다": the integration lists post-norm
hidden-state feedback, and the model card cited there names the layer
norm_output).  The drafter's output hidden state x [M, d] is normalised row by
row with one gamma / beta for all rows.

Reading where the pages are silent: the norm kinds and their definitions are
the ones of the per-state FC normalisation (LayerNorm with biased two-pass
variance and eps inside the root, RMSNorm without mean or beta, NONE = the
un-normalised EAGLE-3 feedback).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .fuse64 import decode_bf16, normalize


def norm_output(X: np.ndarray, kind: int, eps: float, gamma: Optional[np.ndarray],
                beta: Optional[np.ndarray]) -> np.ndarray:
    """Post-norm feedback of one drafter output [M, d], float64.  gamma None
    means ones, beta None zeros (beta is used by LayerNorm only)."""
    return normalize(X, kind, eps, gamma, beta)


def norm_output_bits(x_bits: np.ndarray, kind: int, eps: float, gamma_bits: Optional[np.ndarray],
                     beta_bits: Optional[np.ndarray]) -> np.ndarray:
    """norm_output on bfloat16 bit patterns."""
    g = None if gamma_bits is None else decode_bf16(gamma_bits)
    b = None if beta_bits is None else decode_bf16(beta_bits)
    return norm_output(decode_bf16(x_bits), kind, eps, g, b)
