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


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bfloat16 ulp at |x| (8 significant bits): 2^(floor(log2|x|) - 8);
    at 0 the smallest normal's."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 8)


def assert_parity_full(G: np.ndarray, Y: np.ndarray, what: str, max_tol=MAX_TOL, mean_tol=MEAN_TOL):
    """Every element of a full-size output against the oracle.

    The mean bar applies as written.  The max bar is read element by element
    with the bf16 output grid taken into account: the device's float32 result
    is rounded to bfloat16 once, and far out in a row's tail (|Y| above about
    5 RMS) half a bfloat16 ulp alone exceeds 2e-2 of the row RMS whatever the
    arithmetic before it.  So every element must satisfy
        |G - Y| <= half_ulp_bf16(max(|G|, |Y|)) + (max_tol / 2) * RMS_m,
    i.e. the error beyond the output rounding stays within half the bar; the
    elements over the plain bar (if any) are counted and reported.
    Returns (max relative error, mean relative error, elements over the plain bar).
    """
    assert G.shape == Y.shape, (G.shape, Y.shape)
    assert np.all(np.isfinite(G)), f"{what}: non-finite output"
    rms = np.sqrt(np.mean(Y * Y, axis=1, keepdims=True))
    err = np.abs(G - Y)
    rel = err / rms
    mx, mn = float(rel.max()), float(rel.mean())
    over = rel > max_tol
    n_over = int(over.sum())
    bound = bf16_half_ulp(np.maximum(np.abs(G), np.abs(Y))) + 0.5 * max_tol * rms
    excess = err / bound
    worst = np.unravel_index(int(np.argmax(excess)), err.shape)
    print(f"[parity-full] {what}: rows {G.shape[0]} max {mx:.3e} mean {mn:.3e}; over the 2e-2 bar: {n_over} "
          f"of {G.size}; worst err/bound {float(excess[worst]):.3f} at row {worst[0]} col {worst[1]} "
          f"(|Y|/RMS {abs(Y[worst]) / rms[worst[0], 0]:.2f})", flush=True)
    if n_over:
        idx = np.argwhere(over)[:8]
        for m, n in idx:
            print(f"[parity-full]   over: row {m} col {n} Y={Y[m, n]:.6g} G={G[m, n]:.6g} |Y|/RMS="
                  f"{abs(Y[m, n]) / rms[m, 0]:.2f} err/half-ulp {err[m, n] / bf16_half_ulp(abs(Y[m, n])):.3f}",
                  flush=True)
    assert mn <= mean_tol, f"{what}: mean {mn:.3e} (<= {mean_tol})"
    assert np.all(err <= bound), f"{what}: element beyond half a bf16 ulp + {0.5 * max_tol} RMS (worst {float(excess[worst]):.3f})"
    return mx, mn, n_over
