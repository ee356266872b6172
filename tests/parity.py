"""Helpers shared by the GPU parity tests: moving generator bits to the GPU,
running the oracle on the same bits, and the row-RMS-normalised error metric.

Tolerance (derived from the arithmetic, see the design notes): the device
rounds the normalised activations (or the folded weight) and the output to
bfloat16 and accumulates in float32.  Two bfloat16 roundings of relative size
2^-9 give a per-element error of about 2e-3 of the row RMS at worst and far
less on average; the bars below leave a 2-4x margin:
    max_{m,n} |G - Y| / RMS_m  <= 2e-2,    mean_{m,n} |G - Y| / RMS_m <= 4e-3,
with RMS_m = sqrt(mean_n Y[m, n]^2) of the oracle row.
"""

from __future__ import annotations

import numpy as np

MAX_TOL = 2e-2
MEAN_TOL = 4e-3


def to_dev(bits: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def unpack_folded(tiles, d: int) -> np.ndarray:
    """The folded weight's tiles back to W' [3d, d], from the layout the C
    header documents: tile (n/16, k/32), lane 16*((k%32)/8) + n%16, slot k%8."""
    t = np.asarray(tiles).reshape(d // 16, 3 * d // 32, 4, 16, 8)  # nb, kstep, kgroup, ncol, kk
    return np.transpose(t, (1, 2, 4, 0, 3)).reshape(3 * d, d)


def bf16_to_f64(t) -> np.ndarray:
    """Device bf16 tensor -> float64 numpy (exact)."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def row_rms_errors(G: np.ndarray, Y: np.ndarray):
    rms = np.sqrt(np.mean(Y * Y, axis=1, keepdims=True))
    rel = np.abs(G - Y) / rms
    return float(rel.max()), float(rel.mean())


def assert_parity(G: np.ndarray, Y: np.ndarray, what: str, max_tol=MAX_TOL, mean_tol=MEAN_TOL):
    assert G.shape == Y.shape, (G.shape, Y.shape)
    assert np.all(np.isfinite(G)), f"{what}: non-finite output"
    mx, mn = row_rms_errors(G, Y)
    print(f"[parity] {what}: max {mx:.3e} mean {mn:.3e}", flush=True)
    assert mx <= max_tol and mn <= mean_tol, f"{what}: max {mx:.3e} (<= {max_tol}), mean {mn:.3e} (<= {mean_tol})"
    return mx, mn


class DevInputs:
    """Device copies of a synth.Inputs instance."""

    def __init__(self, inp, device="cuda"):
        self.inp = inp
        self.M, self.d = inp.M, inp.d
        self.h = [to_dev(x, device) for x in inp.h]
        self.gamma = [to_dev(x, device) for x in inp.gamma]
        self.beta = None if inp.beta is None else [to_dev(x, device) for x in inp.beta]
        self.W = to_dev(inp.W, device)
        self.bias = None if inp.bias is None else to_dev(inp.bias, device)


def sample_rows(M: int, k: int = 48, seed: int = 0) -> np.ndarray:
    """Rows checked at full size: the first and last 8 (tile edges and the
    ragged tail) plus a seeded random sample."""
    if M <= k + 16:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(8, M - 8), size=k, replace=False)
    return np.unique(np.concatenate([np.arange(8), mid, np.arange(M - 8, M)]))
