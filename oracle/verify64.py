"""Oracle of the speculative-decoding verify / accept step.

TEST INFRASTRUCTURE.  Only the tests (and the smoke check / bench baseline)
may import this module.  It shares no code with the device path.

What the step computes, from the invariant stated in the speculative-decoding
lesson (factory.pai-world.com/.../15-speculative-decoding-eagle3, section
"불변식: Leviathan 거부 샘플링"): with p the drafter's next-token distribution
and q the verifier's, a draft token d is kept with probability
min(1, q(d) / p(d)); after a rejection the emitted token is drawn from the
positive part of q - p, normalised; the emitted token then follows q, however
poor p is.  N drafts are checked against one verifier pass that yields
q_1 .. q_{N+1}: left to right, the first rejection (position j) emits a token
from the residual of (q_j, p_j) and ends the step; when all N are kept, one
more (bonus) token is drawn from q_{N+1}.

How each part is read (the pages state the rule, not its arithmetic):

* randomness is an input: u_acc [B, N] for the keep decisions and u_res [B]
  for the emitted token, uniforms in [0, 1);
* keep  <=>  u * p(d) < q(d), the product rounded to float32.  For p(d) > 0
  this is u < q(d) / p(d), i.e. the keep probability min(1, q/p), written
  without a division.  A draft with p(d) = 0 (one the drafter could not have
  drawn) is kept exactly when q(d) > 0, so a token the verifier gives zero
  probability is never kept.  A draft id outside [0, V) counts as
  p(d) = q(d) = 0: rejected;
* the residual weights are max(q_j - p_j, 0), the difference rounded to
  float32 (a NaN difference stays NaN); when every one of them is zero (possible only when q_j <= p_j
  everywhere, i.e. q_j = p_j for two distributions, where a rejection needs
  q(d) = p(d) = 0) the token is drawn from q_j itself, which is what the
  invariant asks for;
* a token is drawn from weights w by inverse CDF in token order, in exact
  arithmetic: the smallest t with w_0 + ... + w_t > u_res * (w_0 + ... +
  w_{V-1}).  Every float32 value in [0, 1] is an integer multiple of 2^-149,
  so the sums are exact integers here (any summation order gives the same
  t); the picked token always has w_t > 0;
* a row whose weights are all zero, contain a value outside [0, 1] (or NaN),
  or a u_res outside [0, 1), gives next_token = -1 (no token).
"""

from __future__ import annotations

from itertools import accumulate

import numpy as np

_SCALE = 1 << 149  # 2^149: one step of float32 at the bottom of its range


def _fixed(w: float) -> int:
    """Exact integer w * 2^149 of a float32 value w >= 0."""
    num, den = float(w).as_integer_ratio()
    return num * (_SCALE // den)


def inverse_cdf(weights, u: float) -> int:
    """Smallest t with sum(weights[:t+1]) > u * sum(weights), exactly;
    -1 when the weights are all zero, any is outside [0, 1] or NaN, or u is
    outside [0, 1)."""
    w = np.asarray(weights, dtype=np.float32)
    u = float(np.float32(u))
    if not (0.0 <= u < 1.0):
        return -1
    if not _valid(w):
        return -1
    ints = [_fixed(x) for x in w.tolist()]
    total = sum(ints)
    if total == 0:
        return -1
    un, ud = u.as_integer_ratio()
    # S_t > u * total  <=>  S_t * ud > un * total  (all integers)
    rhs = un * total
    for t, s in enumerate(accumulate(ints)):
        if s * ud > rhs:
            return t
    raise AssertionError("unreachable: the full sum exceeds u * total for u < 1")


def _valid(w) -> bool:
    """Every weight in [0, 1] (False if any is NaN)."""
    return bool(np.all((w >= 0) & (w <= 1)))


def keep_draft(p_d, q_d, u) -> bool:
    """u * p(d) < q(d) with the product rounded to float32."""
    return bool(np.float32(u) * np.float32(p_d) < np.float32(q_d))


def verify_accept(p: np.ndarray, q: np.ndarray, draft: np.ndarray, u_acc: np.ndarray, u_res: np.ndarray):
    """Batched verify step.

    p [B, N, V] and q [B, N+1, V]: float32 probabilities; draft [B, N] int
    token ids; u_acc [B, N], u_res [B]: float32 uniforms in [0, 1).
    Returns (n_accepted [B] int32, next_token [B] int32): the number of drafts
    kept and the token emitted after them (the residual's at the first
    rejection, else the bonus from q_{N+1}; -1 for an invalid row).
    """
    p = np.asarray(p, dtype=np.float32)
    q = np.asarray(q, dtype=np.float32)
    draft = np.asarray(draft, dtype=np.int64)
    u_acc = np.asarray(u_acc, dtype=np.float32)
    u_res = np.asarray(u_res, dtype=np.float32)
    B, N, V = p.shape
    n_acc = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        j = N
        for i in range(N):
            t = int(draft[b, i])
            inside = 0 <= t < V
            pd = p[b, i, t] if inside else np.float32(0)
            qd = q[b, i, t] if inside else np.float32(0)
            if not keep_draft(pd, qd, u_acc[b, i]):
                j = i
                break
        n_acc[b] = j
        if j < N:
            w = np.maximum(q[b, j] - p[b, j], np.float32(0))  # NaN stays NaN
            if _valid(w) and not np.any(w > 0):
                w = q[b, j]
        else:
            w = q[b, N]
        nxt[b] = inverse_cdf(w, u_res[b])
    return n_acc, nxt
