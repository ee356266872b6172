"""Seeded generator: draws every tensor with numpy and rounds it to bfloat16.

Recipe (the same for every workload unless the workload overrides a field):

* h_s[m, c] = scale_s * z[m, c] + o_s[c], z ~ N(0, 1) i.i.d., o_s[c] ~ N(0, offset_std_s)
  shared by all tokens; optional outlier channels: n_outliers distinct channels
  per state whose whole column is multiplied by outlier_mult after scale+offset;
* gamma_s ~ N(1, 0.1), beta_s ~ N(0, 0.05), W ~ N(0, 1/sqrt(3d)), bias ~ N(0, 0.01)
  (N(a, b) means mean a, standard deviation b);
* numpy Generator(PCG64) seeded with SeedSequence(seed).spawn(...), one child
  stream per tensor, so changing one tensor's shape never shifts another's draws;
  standard normals are drawn in float32 (numpy's float32 ziggurat) and the
  affine recipe is evaluated in float32;
* a workload with several M draws its largest M once and every smaller M is the
  leading rows of it (M=4093 is a prefix of M=4096).

Rounding to bfloat16 is round-to-nearest-even of the float32 value, done with
integer operations on the bit pattern.  The arrays handed out are the raw
uint16 bit patterns, which both the oracle and the device path decode by
themselves.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from .workloads import CONFIGS, Workload

# child-stream indices of SeedSequence.spawn
_S_Z = (0, 1, 2)
_S_OFFSET = 3
_S_OUTLIER = 4
_S_GAMMA = 5
_S_BETA = 6
_S_W = 7
_S_BIAS = 8
_N_STREAMS = 9

_CHUNK_ELEMS = 1 << 22


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of x rounded to nearest, ties to even.

    x is taken as float32 (values given in float64 are first rounded to
    float32).  bfloat16 is the top half of a float32: adding 0x7FFF plus the
    lowest kept bit and truncating rounds half to even; a carry out of the
    mantissa bumps the exponent, which is the correct result.  Values here are
    finite and far from the overflow range.
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 values of x (via float32), returned as float64."""
    return bits_to_f32(bf16_bits(x)).astype(np.float64)


def _to_bits(x: np.ndarray) -> np.ndarray:
    return bf16_bits(x)


@dataclass
class Inputs:
    """bfloat16 bit patterns of one problem instance."""

    d: int
    M: int
    h: List[np.ndarray]              # 3 x uint16 [M, d], order low, mid, high
    gamma: List[np.ndarray]          # 3 x uint16 [d]
    beta: Optional[List[np.ndarray]]  # 3 x uint16 [d] or None
    W: np.ndarray                    # uint16 [3d, d], row k multiplies concat column k
    bias: Optional[np.ndarray]       # uint16 [d] or None

    def rows(self, M: int) -> "Inputs":
        """The leading M tokens of this instance (parameters shared)."""
        if M > self.M:
            raise ValueError("cannot grow an instance")
        return Inputs(self.d, M, [x[:M] for x in self.h], self.gamma, self.beta, self.W, self.bias)


def _normal_rows(rng: np.random.Generator, rows: int, cols: int, std: float,
                 mean: float = 0.0) -> np.ndarray:
    """Draw [rows, cols] N(mean, std) in row chunks and return bf16 bits."""
    out = np.empty((rows, cols), dtype=np.uint16)
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        z = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        out[r0:r1] = _to_bits(np.float32(mean) + np.float32(std) * z)
    return out


def make_inputs(cfg, M: Optional[int] = None, *, extra_offset: Sequence[float] = (0.0, 0.0, 0.0),
                with_weights: bool = True) -> Inputs:
    """Generate the inputs of a workload.

    cfg: a workload id (1..5) or a Workload instance.
    M: number of tokens; defaults to the workload's largest M.  Rows are the
       leading rows of the workload's largest-M draw when M <= max_M.
    extra_offset: a constant added to every element of state s before
       rounding (used by the shared DC-offset stress case).
    with_weights: skip W (returns a zero-size array) when only activations
       are needed.
    """
    w: Workload = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    d = w.d
    M = w.max_M if M is None else M
    # Draws are sequential per stream, so the first M rows are the same
    # whatever the largest M is: drawing only M rows keeps the prefix rule.
    rows_drawn = M
    ss = np.random.SeedSequence(w.seed)
    kids = ss.spawn(_N_STREAMS)
    rng = [np.random.Generator(np.random.PCG64(k)) for k in kids]

    offsets = [rng[_S_OFFSET].standard_normal(d, dtype=np.float32) * np.float32(w.offset_std[s])
               for s in range(3)]
    outlier_cols = []
    for s in range(3):
        if w.n_outliers > 0:
            outlier_cols.append(np.sort(rng[_S_OUTLIER].choice(d, size=w.n_outliers, replace=False)))
        else:
            outlier_cols.append(np.zeros(0, dtype=np.int64))

    h = []
    for s in range(3):
        g = rng[_S_Z[s]]
        out = np.empty((M, d), dtype=np.uint16)
        step = max(1, _CHUNK_ELEMS // d)
        r0 = 0
        while r0 < rows_drawn:
            r1 = min(rows_drawn, r0 + step)
            z = g.standard_normal((r1 - r0, d), dtype=np.float32)
            x = np.float32(w.scales[s]) * z + offsets[s][None, :]
            if w.n_outliers > 0:
                x[:, outlier_cols[s]] *= np.float32(w.outlier_mult)
            if extra_offset[s] != 0.0:
                x += np.float32(extra_offset[s])
            out[r0:r1] = _to_bits(x)
            r0 = r1
        h.append(out)

    gamma = [_to_bits(np.float32(w.gamma_mean) + np.float32(w.gamma_std)
                      * rng[_S_GAMMA].standard_normal(d, dtype=np.float32)) for _ in range(3)]
    beta = ([_to_bits(np.float32(w.beta_std) * rng[_S_BETA].standard_normal(d, dtype=np.float32))
             for _ in range(3)] if w.has_beta else None)
    if with_weights:
        W = _normal_rows(rng[_S_W], 3 * d, d, w.w_std)
    else:
        W = np.zeros((0, d), dtype=np.uint16)
    bias = (_to_bits(np.float32(w.bias_std) * rng[_S_BIAS].standard_normal(d, dtype=np.float32))
            if w.has_bias else None)
    return Inputs(d, M, h, gamma, beta, W, bias)


def custom_workload(d: int, Ms, seed_tag: int, *, scales=(1.0, 4.0, 16.0), offset_std=(0.5, 0.5, 0.5),
                    n_outliers: int = 0, outlier_mult: float = 1.0, has_beta: bool = True,
                    has_bias: bool = True, norms=((1, 1e-5),)) -> Workload:
    """A workload with the default recipe at an arbitrary size (edge cases).

    seed_tag keeps edge-case seeds apart from the five named workloads.
    """
    return Workload(1000 + seed_tag, f"custom{seed_tag}_d{d}", d, tuple(Ms), tuple(norms), tuple(scales),
                    tuple(offset_std), n_outliers, outlier_mult, has_beta, has_bias)


def make_embed_inputs(M: int, d: int, vocab: int, seed: int, n_bad: int = 0):
    """Inputs of the drafter-input concatenation: token ids int32 [M] uniform
    over [0, vocab), of which n_bad spread positions are replaced by ids
    outside the table (alternately -1 - k and vocab + k); an embedding table
    bf16 [vocab, d] ~ N(0, 0.02); a fused feature bf16 [M, d] ~ N(0, 1).
    Returns (tokens, embed_bits, fused_bits)."""
    s_tok, s_emb, s_fus = np.random.SeedSequence(seed).spawn(3)
    tokens = np.random.Generator(np.random.PCG64(s_tok)).integers(0, vocab, size=M, dtype=np.int64)
    for k, pos in enumerate(np.linspace(0, M - 1, num=min(n_bad, M), dtype=np.int64)):
        tokens[pos] = -1 - k if k % 2 == 0 else vocab + k
    rng_e = np.random.Generator(np.random.PCG64(s_emb))
    embed = bf16_bits(rng_e.standard_normal((vocab, d), dtype=np.float32) * np.float32(0.02))
    rng_f = np.random.Generator(np.random.PCG64(s_fus))
    fused = bf16_bits(rng_f.standard_normal((M, d), dtype=np.float32))
    return tokens.astype(np.int32), embed, fused
