"""Oracle of the drafter-input concatenation.

TEST INFRASTRUCTURE.  Only the tests and the bench may import this module.
It shares no code with the device path.

What it computes (EAGLE-3 paper summary, honbul.tistory.com/173, section
"EAGLE-3가 바꾼 것 2": the low, middle and high features are fused into one
feature, and the embedding of the token sampled just before is joined to it
before the draft model).  Readings where the page is silent: the two are
concatenated, not summed, into one [M, 2d] drafter input row, embedding
first; a token id outside the table gives a zero embedding half and is
counted.  It is byte work, so the oracle moves bit patterns and nothing is
rounded.
"""

from __future__ import annotations

import numpy as np


def embed_concat(tokens: np.ndarray, embed_bits: np.ndarray, fused_bits: np.ndarray):
    """dst [M, 2d] uint16 with dst[m] = embed[tokens[m]] followed by fused[m]
    (zeros for the first half when tokens[m] is outside [0, vocab)); returns
    (dst, number of such tokens)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    embed = np.asarray(embed_bits, dtype=np.uint16)
    fused = np.asarray(fused_bits, dtype=np.uint16)
    vocab, d = embed.shape
    ok = (tokens >= 0) & (tokens < vocab)
    left = np.zeros((tokens.shape[0], d), dtype=np.uint16)
    left[ok] = embed[tokens[ok]]
    return np.concatenate([left, fused], axis=1), int(np.count_nonzero(~ok))
