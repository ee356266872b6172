"""Oracle of the speculative-decoding verify / accept step.

TEST INFRASTRUCTURE.  Only the tests may import this module.  It shares no
code with the device path.

What it computes (speculative-decoding lesson,
factory.pai-world.com/.../15-speculative-decoding-eagle3, section "불변식:
Leviathan 거부 샘플링"): a draft token d drawn from the drafter's
distribution p is kept with probability min(1, q(d) / p(d)), q being the
verifier's distribution; on rejection the token is drawn from the positive
part of q - p, normalised, and the result follows q whatever p is.  With N
drafts checked by one verifier pass (q_1 .. q_{N+1}), the drafts are taken
left to right: the first rejection at position j emits a token from the
residual of (q_j, p_j) and stops; if all N are kept, a bonus token is drawn
from q_{N+1}.

Readings where the pages are silent (listed in the design notes):

* randomness is an input: u_acc [B, N] for the keep decisions and one u_res [B]
  for the emitted token, each in [0, 1);
* the keep decision is u < min(1, q(d) / p(d)) evaluated in float32 (the
  device's precision), and a draft with p(d) <= 0 is kept;
* the emitted token is drawn by inverse CDF over the token index order: the
  smallest t whose running sum of weights exceeds u_res times their total; the
  weights are max(q - p, 0) (unnormalised; normalising does not change t) and,
  when they are all zero (q = p on that row), q itself.  Sums here are float64.
"""

from __future__ import annotations

import numpy as np


def inverse_cdf(weights: np.ndarray, u: float) -> int:
    """Smallest index whose inclusive running sum of `weights` exceeds u * total."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    target = float(u) * c[-1]
    return int(np.searchsorted(c, target, side="right"))


def verify_accept(p: np.ndarray, q: np.ndarray, draft: np.ndarray, u_acc: np.ndarray, u_res: np.ndarray):
    """Batched verify step.

    p [B, N, V] and q [B, N+1, V]: float32 probabilities; draft [B, N] int
    token ids; u_acc [B, N], u_res [B]: float32 uniforms in [0, 1).
    Returns (n_accepted [B] int32, next_token [B] int32): the number of drafts
    kept and the token emitted after them (the residual's at the first
    rejection, else the bonus from q_{N+1}).
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
            pd = p[b, i, draft[b, i]]
            qd = q[b, i, draft[b, i]]
            keep = pd <= np.float32(0) or u_acc[b, i] < min(np.float32(1), np.float32(qd / pd))
            if not keep:
                j = i
                break
        n_acc[b] = j
        if j < N:
            w = np.maximum(q[b, j] - p[b, j], np.float32(0))
            if not np.any(w > 0):
                w = q[b, j]
        else:
            w = q[b, N]
        nxt[b] = inverse_cdf(w, u_res[b])
    return n_acc, nxt
