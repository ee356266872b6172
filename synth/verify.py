"""Seeded inputs of the speculative-decoding verify step.

Draws only: next-token distributions for the drafter (p) and the verifier
(q), draft tokens drawn from p, and the uniforms the step consumes.  The
distributions are softmaxes of shared seeded logits plus independent
per-model noise (so the two models agree often but not always, as a draft
head trained on the verifier's features does); none of the step's arithmetic
(keep decisions, residuals, inverse CDF) is here.

Recipe: base logits ~ N(0, temp) per (sequence, position, token); drafter
logits = base + N(0, spread), verifier logits = base + N(0, spread); both
softmaxed in float64 and stored as float32.  Drafts d_i ~ p_i by numpy's
sampler; u_acc, u_res ~ U[0, 1) as float32.  The verifier has N + 1
positions (the last gives the bonus token).
"""

from __future__ import annotations

import numpy as np


def _softmax(x: np.ndarray) -> np.ndarray:
    z = x - x.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def make_verify_inputs(B: int, N: int, V: int, seed: int, temp: float = 3.0, spread: float = 1.0):
    """Returns (p [B, N, V] f32, q [B, N+1, V] f32, draft [B, N] i32, u_acc [B, N] f32, u_res [B] f32)."""
    s_base, s_p, s_q, s_d, s_u = np.random.SeedSequence(seed).spawn(5)
    base = np.random.Generator(np.random.PCG64(s_base)).standard_normal((B, N + 1, V)) * temp
    pl = base[:, :N] + np.random.Generator(np.random.PCG64(s_p)).standard_normal((B, N, V)) * spread
    ql = base + np.random.Generator(np.random.PCG64(s_q)).standard_normal((B, N + 1, V)) * spread
    p64 = _softmax(pl)
    q = _softmax(ql).astype(np.float32)
    p = p64.astype(np.float32)
    rng_d = np.random.Generator(np.random.PCG64(s_d))
    draft = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        for i in range(N):
            draft[b, i] = rng_d.choice(V, p=p64[b, i] / p64[b, i].sum())
    rng_u = np.random.Generator(np.random.PCG64(s_u))
    u_acc = rng_u.random((B, N), dtype=np.float32)
    u_res = rng_u.random(B, dtype=np.float32)
    return p, q, draft, u_acc, u_res
