"""fp64 CPU oracle of the EAGLE-3.1 normalized multi-layer feature fusion.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the bench's
cpu_baseline leg may import this module.  It shares no code with the device
path: it decodes the bfloat16 bit patterns itself and computes everything in
float64 with numpy, in the order the pages state the method.

What it computes (sources, cited by page and section):

* EAGLE 3.1 explainer, llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html
  - section "EAGLE-3의 다층 특성 융합 구조": three target hidden states (early,
    middle, late layer) are concatenated and an FC layer projects the
    concatenation to the draft head's input width;
  - section "FC 정규화: EAGLE 3.1의 핵심 수정": EAGLE 3.1 applies a LayerNorm
    to each of the three states on its own before the concatenation, the
    concatenation order stays early, middle, late; the LayerNorm parameters
    are said to be absorbed into the FC (the fold below).
* vLLM EAGLE 3.1 release post, devlery.com/blog/vllm-eagle31-attention-drift,
  section "EAGLE 3.1이 바꾼 것은 작지만 낮은 계층입니다": the normalisation is
  described as an RMSNorm per target hidden state, hence the RMS variant.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* LayerNorm: biased variance (divide by d) from two passes (mean first, then
  the mean of squared deviations), eps inside the square root, per-state
  affine gamma_s / beta_s;
* RMSNorm: x * (mean(x^2) + eps)^(-1/2) * gamma_s, no mean, no beta;
* NONE: the state is used as is (EAGLE-3 fusion);
* W is [3d, d] with row k multiplying column k of the concatenation, so
  Y = X @ W + bias; rows [s*d, (s+1)*d) of W belong to state s.
"""

from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

NORM_NONE = 0
NORM_LN = 1
NORM_RMS = 2


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float64 values."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def row_stats(X: np.ndarray, kind: int, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row (mu, rstd) of one hidden state X [M, d] in float64.

    LayerNorm: mu = mean(x), var = mean((x - mu)^2) (two passes, biased),
    rstd = 1 / sqrt(var + eps).  RMSNorm: mu = 0, rstd = 1 / sqrt(mean(x^2) + eps).
    NONE: mu = 0, rstd = 1.
    """
    X = np.asarray(X, dtype=np.float64)
    M = X.shape[0]
    if kind == NORM_LN:
        mu = X.mean(axis=1)
        var = ((X - mu[:, None]) ** 2).mean(axis=1)
        return mu, 1.0 / np.sqrt(var + eps)
    if kind == NORM_RMS:
        ms = (X * X).mean(axis=1)
        return np.zeros(M), 1.0 / np.sqrt(ms + eps)
    if kind == NORM_NONE:
        return np.zeros(M), np.ones(M)
    raise ValueError(f"unknown norm kind {kind}")


def normalize(X: np.ndarray, kind: int, eps: float, gamma: Optional[np.ndarray],
              beta: Optional[np.ndarray]) -> np.ndarray:
    """Normalise one hidden state [M, d] (explainer, FC-normalisation section;
    release post for the RMS form).  gamma None means ones, beta None zeros."""
    X = np.asarray(X, dtype=np.float64)
    if kind == NORM_NONE:
        return X.copy()
    mu, r = row_stats(X, kind, eps)
    g = np.ones(X.shape[1]) if gamma is None else np.asarray(gamma, dtype=np.float64)
    if kind == NORM_LN:
        b = np.zeros(X.shape[1]) if beta is None else np.asarray(beta, dtype=np.float64)
        return (X - mu[:, None]) * r[:, None] * g[None, :] + b[None, :]
    # RMS: no mean subtraction, no shift
    return X * r[:, None] * g[None, :]


def fuse(H: Sequence[np.ndarray], kind: int, eps: float, gammas: Optional[Sequence[np.ndarray]],
         betas: Optional[Sequence[np.ndarray]], W: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """Y = [norm(h_low) | norm(h_mid) | norm(h_high)] @ W + bias, float64.

    H: three float64 arrays [M, d] (low, mid, high).  W: float64 [3d, d].
    The concatenation is materialised here on purpose: this is the plain
    definition, not the fast path.
    """
    if len(H) != 3:
        raise ValueError("need exactly three hidden states")
    parts = []
    for s in range(3):
        g = None if gammas is None else gammas[s]
        b = None if betas is None else betas[s]
        parts.append(normalize(H[s], kind, eps, g, b))
    X = np.concatenate(parts, axis=1)
    Y = X @ np.asarray(W, dtype=np.float64)
    if bias is not None:
        Y = Y + np.asarray(bias, dtype=np.float64)[None, :]
    return Y


def fuse_bits(inp, kind: int, eps: float, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """The oracle on a synth.Inputs instance (bfloat16 bit patterns).

    rows: optional token indices; the step is row independent, so the result
    for a subset of tokens is the subset of the full result.
    """
    H = [decode_bf16(h if rows is None else h[rows]) for h in inp.h]
    gam = [decode_bf16(g) for g in inp.gamma]
    bet = None if inp.beta is None else [decode_bf16(b) for b in inp.beta]
    W = decode_bf16(inp.W)
    bias = None if inp.bias is None else decode_bf16(inp.bias)
    return fuse(H, kind, eps, gam, bet, W, bias)


# ---------------------------------------------------------------------------
# The fold: the explainer's FC-normalisation section says the LayerNorm
# parameters are absorbed into the FC layer.  Written out: with
# W'_s = diag(gamma_s) W_s, u_s = 1^T W'_s and c = bias + sum_s beta_s^T W_s,
#   Y = sum_s rstd_s * (h_s W'_s - mu_s u_s) + c,
# which equals fuse() in exact arithmetic.
# ---------------------------------------------------------------------------


def fold_prepare(kind: int, gammas: Optional[Sequence[np.ndarray]], betas: Optional[Sequence[np.ndarray]],
                 W: np.ndarray, bias: Optional[np.ndarray], round_w=None):
    """Return (Wf [3d, d], u [3, d], c [d]) of the fold, float64.

    round_w: optional function applied to W' before u is formed (the device
    stores W' in bfloat16; u must be the column sums of the stored W').
    """
    W = np.asarray(W, dtype=np.float64)
    d = W.shape[1]
    Wf = W.copy()
    if kind in (NORM_LN, NORM_RMS) and gammas is not None:
        for s in range(3):
            Wf[s * d:(s + 1) * d] *= np.asarray(gammas[s], dtype=np.float64)[:, None]
    if round_w is not None:
        Wf = round_w(Wf)
    u = np.stack([Wf[s * d:(s + 1) * d].sum(axis=0) for s in range(3)])
    c = np.zeros(d) if bias is None else np.asarray(bias, dtype=np.float64).copy()
    if kind == NORM_LN and betas is not None:
        for s in range(3):
            c += np.asarray(betas[s], dtype=np.float64) @ W[s * d:(s + 1) * d]
    return Wf, u, c


def fold_apply(H: Sequence[np.ndarray], kind: int, eps: float, Wf: np.ndarray, u: np.ndarray,
               c: np.ndarray) -> np.ndarray:
    """Y = sum_s rstd_s * (h_s W'_s - mu_s u_s) + c on raw (un-normalised) states."""
    d = Wf.shape[1]
    Y = np.zeros((H[0].shape[0], d)) + c[None, :]
    for s in range(3):
        X = np.asarray(H[s], dtype=np.float64)
        mu, r = row_stats(X, kind, eps)
        P = X @ Wf[s * d:(s + 1) * d]
        Y += r[:, None] * (P - mu[:, None] * u[s][None, :])
    return Y


def round_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of float64 x, ties to even (oracle's own copy).

    Used to state what the device's stored W' = bf16(gamma * W) must be:
    gamma and W are bfloat16, so gamma * W is exact in float64 and its
    rounding has one correct answer.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)
