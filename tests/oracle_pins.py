"""Pin checks for the fp64 oracle, written against what the pages and the
mathematics fix rather than against the oracle itself.

Every check takes the fusion function under test (signature of
oracle.fuse) so the same checks can be pointed at deliberately broken
variants (tests/test_oracle_mutants.py): a plausible slip in the oracle must
make at least one of them fail.

Sources: EAGLE 3.1 explainer (llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html),
sections "EAGLE-3의 다층 특성 융합 구조" (the magnitude imbalance between early and
late states is the problem) and "FC 정규화: EAGLE 3.1의 핵심 수정" (per-state
LayerNorm before the FC, same scale for the three states, EAGLE-3 = no norm);
vLLM EAGLE 3.1 release post (devlery.com/blog/vllm-eagle31-attention-drift),
section "EAGLE 3.1이 바꾼 것은 작지만 낮은 계층입니다" (per-state RMSNorm).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

NORM_NONE, NORM_LN, NORM_RMS = 0, 1, 2
NORM_BY_NAME = {"none": NORM_NONE, "layernorm": NORM_LN, "rmsnorm": NORM_RMS}

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_hand_example():
    with open(os.path.join(GOLDEN, "hand_d4.json")) as f:
        g = json.load(f)
    d = g["d"]
    H = [np.array(g["h_low"], float), np.array(g["h_mid"], float), np.array(g["h_high"], float)]
    W = np.zeros((3 * d, d))
    for k, n, v in g["W_nonzero"]:
        W[k, n] = v
    bias = np.array(g["bias"], float)
    env = {"sqrt": math.sqrt}
    cases = []
    for c in g["cases"]:
        exp = np.array([[eval(e, {"__builtins__": {}}, env) for e in row] for row in c["expected"]])
        gam = None if c["gamma"] is None else [np.array(x, float) for x in c["gamma"]]
        bet = None if c["beta"] is None else [np.array(x, float) for x in c["beta"]]
        cases.append((NORM_BY_NAME[c["norm"]], gam, bet, exp))
    return H, W, bias, cases


def check_hand_example(fuse_fn, tol=1e-12) -> bool:
    """Closed forms of tests/golden/hand_d4.json (eps = 0)."""
    H, W, bias, cases = load_hand_example()
    for kind, gam, bet, exp in cases:
        Y = fuse_fn(H, kind, 0.0, gam, bet, W, bias)
        if not np.allclose(Y, exp, rtol=0, atol=tol):
            return False
    return True


def _ident_params(d):
    return [np.ones(d)] * 3, [np.zeros(d)] * 3


def normalized_segments(fuse_fn, H, kind, eps):
    """Recover each normalised state through the FC by choosing W = [I;0;0],
    [0;I;0], [0;0;I] (gamma = 1, beta = 0, no bias)."""
    d = H[0].shape[1]
    g, b = _ident_params(d)
    out = []
    for s in range(3):
        W = np.zeros((3 * d, d))
        W[s * d:(s + 1) * d] = np.eye(d)
        out.append(fuse_fn(H, kind, eps, g, b, W, None))
    return out


def check_moments(fuse_fn, H, tol=1e-9) -> bool:
    """Normalised moments (closed form): LN at eps = 0 gives mean 0 and
    variance 1 per row and state; at eps > 0 the variance is v / (v + eps);
    RMS at eps = 0 gives mean square 1, at eps > 0 ms / (ms + eps)."""
    for eps in (0.0, 1e-5):
        segs = normalized_segments(fuse_fn, H, NORM_LN, eps)
        for s in range(3):
            X = H[s]
            n = segs[s]
            v = np.var(X, axis=1)  # numpy's population variance
            if np.max(np.abs(n.mean(axis=1))) > tol:
                return False
            target = np.ones_like(v) if eps == 0.0 else v / (v + eps)
            if np.max(np.abs(n.var(axis=1) - target)) > tol:
                return False
        segs = normalized_segments(fuse_fn, H, NORM_RMS, eps)
        for s in range(3):
            ms = np.mean(H[s] ** 2, axis=1)
            target = np.ones_like(ms) if eps == 0.0 else ms / (ms + eps)
            if np.max(np.abs(np.mean(segs[s] ** 2, axis=1) - target)) > tol:
                return False
    return True


def check_scale_invariance(fuse_fn, H, gam, W, bias, scales=(0.125, 0.5, 2.0, 16.0, 10.0)) -> bool:
    """The point of the FC normalisation is that the magnitude of each state
    no longer matters.  With beta = 0 (LN) or RMS and eps = 0, scaling any one
    state by c > 0 leaves Y unchanged up to float64 rounding; under NONE the
    same scaling must change Y by O(RMS(Y)) (negative control)."""
    d = H[0].shape[1]
    zero_b = [np.zeros(d)] * 3
    for kind in (NORM_LN, NORM_RMS):
        Y = fuse_fn(H, kind, 0.0, gam, zero_b, W, bias)
        rms = np.sqrt(np.mean(Y ** 2))
        for s in range(3):
            for c in scales:
                Hs = list(H)
                Hs[s] = H[s] * c
                Yc = fuse_fn(Hs, kind, 0.0, gam, zero_b, W, bias)
                if np.max(np.abs(Yc - Y)) > 1e-12 * rms:
                    return False
    Y = fuse_fn(H, NORM_NONE, 0.0, None, None, W, bias)
    Hs = list(H)
    Hs[2] = H[2] * 4.0
    Y4 = fuse_fn(Hs, NORM_NONE, 0.0, None, None, W, bias)
    if np.sqrt(np.mean((Y4 - Y) ** 2)) < 0.5 * np.sqrt(np.mean(Y ** 2)):
        return False
    return True


def check_scale_invariance_eps(fuse_fn, H, gam, W, bias, eps=1e-5, scales=(0.25, 4.0, 16.0)) -> bool:
    """With eps > 0 the invariance is not exact, and the deviation has a
    closed form.  LN(c x) = (x - mu) / sqrt(v + eps / c^2), so every
    normalised value of state s in row m grows by the factor
    f_m = sqrt((v_m + eps) / (v_m + eps / c^2)) and, with beta = 0, the output
    moves by exactly (f_m - 1) * Y_s[m, :], where Y_s is state s's own
    contribution (W restricted to its rows, no bias).  The factor is about
    eps / (2 v) * (1 - 1 / c^2)."""
    d = H[0].shape[1]
    zero_b = [np.zeros(d)] * 3
    Y = fuse_fn(H, NORM_LN, eps, gam, zero_b, W, bias)
    for s in range(3):
        v = np.var(H[s], axis=1)
        Wz = np.zeros_like(W)
        Wz[s * d:(s + 1) * d] = W[s * d:(s + 1) * d]
        Ys = fuse_fn(H, NORM_LN, eps, gam, zero_b, Wz, None)
        for c in scales:
            f = np.sqrt((v + eps) / (v + eps / c ** 2))
            Hs = list(H)
            Hs[s] = H[s] * c
            Yc = fuse_fn(Hs, NORM_LN, eps, gam, zero_b, W, bias)
            want = (f - 1.0)[:, None] * Ys
            if np.max(np.abs((Yc - Y) - want)) > 1e-12 * max(1.0, np.max(np.abs(Y))):
                return False
    return True


def brute_force(H, kind, eps, gam, bet, W, bias):
    """Scalar loops: per-state statistics, normalisation, concatenation and the
    FC written element by element (no numpy reductions)."""
    M, d = len(H[0]), len(H[0][0])
    Y = [[0.0] * d for _ in range(M)]
    for m in range(M):
        xcat = []
        for s in range(3):
            row = [float(H[s][m][i]) for i in range(d)]
            if kind == NORM_NONE:
                xcat.extend(row)
                continue
            if kind == NORM_LN:
                mean = 0.0
                for v in row:
                    mean += v
                mean /= d
                var = 0.0
                for v in row:
                    var += (v - mean) * (v - mean)
                var /= d
                r = 1.0 / math.sqrt(var + eps)
                for i in range(d):
                    g = 1.0 if gam is None else float(gam[s][i])
                    b = 0.0 if bet is None else float(bet[s][i])
                    xcat.append((row[i] - mean) * r * g + b)
            else:
                ms = 0.0
                for v in row:
                    ms += v * v
                ms /= d
                r = 1.0 / math.sqrt(ms + eps)
                for i in range(d):
                    g = 1.0 if gam is None else float(gam[s][i])
                    xcat.append(row[i] * r * g)
        for n in range(d):
            acc = 0.0 if bias is None else float(bias[n])
            for k in range(3 * d):
                acc += xcat[k] * float(W[k][n])
            Y[m][n] = acc
    return np.array(Y)


def check_brute_force(fuse_fn, seed=7, d=4, M=2, tol=1e-13) -> bool:
    rng = np.random.default_rng(seed)
    H = [rng.normal(0, sc, (M, d)) + rng.normal(0, 0.5, d) for sc in (1.0, 4.0, 16.0)]
    gam = [rng.normal(1, 0.1, d) for _ in range(3)]
    bet = [rng.normal(0, 0.05, d) for _ in range(3)]
    W = rng.normal(0, (3 * d) ** -0.5, (3 * d, d))
    bias = rng.normal(0, 0.01, d)
    for kind in (NORM_NONE, NORM_LN, NORM_RMS):
        for eps in (0.0, 1e-5):
            b = bet if kind == NORM_LN else None
            Y = fuse_fn(H, kind, eps, gam if kind != NORM_NONE else None, b, W, bias)
            Yb = brute_force(H, kind, eps, gam if kind != NORM_NONE else None, b, W, bias)
            scale = max(1.0, float(np.max(np.abs(Yb))))
            if np.max(np.abs(Y - Yb)) > tol * scale:
                return False
    return True


def check_torch_library(fuse_fn, seed=11, d=64, M=5, tol=1e-12) -> bool:
    """Cross-check against torch's CPU float64 layer_norm / rms_norm and matmul,
    an independent library implementation of the same textbook operations."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(seed)
    H = [rng.normal(0, sc, (M, d)) + rng.normal(0, 0.5, d) for sc in (1.0, 4.0, 16.0)]
    gam = [rng.normal(1, 0.1, d) for _ in range(3)]
    bet = [rng.normal(0, 0.05, d) for _ in range(3)]
    W = rng.normal(0, (3 * d) ** -0.5, (3 * d, d))
    bias = rng.normal(0, 0.01, d)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    for kind, eps in ((NORM_LN, 1e-5), (NORM_RMS, 1e-6), (NORM_NONE, 0.0)):
        parts = []
        for s in range(3):
            if kind == NORM_LN:
                parts.append(F.layer_norm(t(H[s]), (d,), t(gam[s]), t(bet[s]), eps))
            elif kind == NORM_RMS:
                parts.append(F.rms_norm(t(H[s]), (d,), t(gam[s]), eps))
            else:
                parts.append(t(H[s]))
        ref = (torch.cat(parts, dim=1) @ t(W) + t(bias)).numpy()
        Y = fuse_fn(H, kind, eps, gam if kind != NORM_NONE else None, bet if kind == NORM_LN else None, W, bias)
        if np.max(np.abs(Y - ref)) > tol * max(1.0, np.max(np.abs(ref))):
            return False
    return True


def check_none_is_eagle3(fuse_fn, seed=3, d=32, M=6) -> bool:
    """With the norm off the step is EAGLE-3's plain fusion: the FC applied to
    the raw concatenation, i.e. sum_s h_s @ W_s + bias (computed here one
    state block at a time with torch float64, not numpy)."""
    import torch

    rng = np.random.default_rng(seed)
    H = [rng.normal(0, sc, (M, d)) for sc in (1.0, 4.0, 16.0)]
    W = rng.normal(0, 0.1, (3 * d, d))
    bias = rng.normal(0, 0.01, d)
    ref = torch.from_numpy(bias.copy()).expand(M, d).clone()
    for s in range(3):
        ref += torch.from_numpy(H[s]) @ torch.from_numpy(np.ascontiguousarray(W[s * d:(s + 1) * d]))
    Y = fuse_fn(H, NORM_NONE, 0.0, None, None, W, bias)
    return bool(np.max(np.abs(Y - ref.numpy())) <= 1e-12 * np.max(np.abs(ref.numpy())))


def check_segment_order(fuse_fn, seed=5, d=16, M=3) -> bool:
    """The concatenation order is low, mid, high: a W that is zero except in
    the mid block must see only h_mid (changing h_low / h_high leaves Y)."""
    rng = np.random.default_rng(seed)
    H = [rng.normal(0, sc, (M, d)) for sc in (1.0, 4.0, 16.0)]
    W = np.zeros((3 * d, d))
    W[d:2 * d] = rng.normal(0, 0.3, (d, d))
    g, b = _ident_params(d)
    for kind in (NORM_NONE, NORM_LN, NORM_RMS):
        Y = fuse_fn(H, kind, 1e-5, g, b, W, None)
        H2 = [H[0] * 3 + 1, H[1], -H[2] + 2]
        Y2 = fuse_fn(H2, kind, 1e-5, g, b, W, None)
        if np.max(np.abs(Y2 - Y)) > 1e-12:
            return False
        H3 = [H[0], H[1] + rng.normal(0, 1, (M, d)), H[2]]
        if np.max(np.abs(fuse_fn(H3, kind, 1e-5, g, b, W, None) - Y)) < 1e-6:
            return False
    return True


def check_row_independence(fuse_fn, seed=9, d=16, M=7) -> bool:
    """Each token's output depends only on its own three rows: permuting the
    tokens permutes the rows of Y; perturbing one token changes one row."""
    rng = np.random.default_rng(seed)
    H = [rng.normal(0, sc, (M, d)) + 1.0 for sc in (1.0, 4.0, 16.0)]
    gam = [rng.normal(1, 0.1, d) for _ in range(3)]
    bet = [rng.normal(0, 0.05, d) for _ in range(3)]
    W = rng.normal(0, 0.2, (3 * d, d))
    bias = rng.normal(0, 0.01, d)
    for kind in (NORM_LN, NORM_RMS, NORM_NONE):
        Y = fuse_fn(H, kind, 1e-5, gam, bet, W, bias)
        perm = rng.permutation(M)
        Yp = fuse_fn([h[perm] for h in H], kind, 1e-5, gam, bet, W, bias)
        if np.max(np.abs(Yp - Y[perm])) > 1e-12:
            return False
        H2 = [h.copy() for h in H]
        H2[1][3] += rng.normal(0, 1, d)
        Y2 = fuse_fn(H2, kind, 1e-5, gam, bet, W, bias)
        changed = np.max(np.abs(Y2 - Y), axis=1) > 1e-12
        if not (changed[3] and changed.sum() == 1):
            return False
    return True


def check_fold_identity(fuse_fn, fold_prepare, fold_apply, seed=13, d=32, M=9) -> bool:
    """The explainer says the LayerNorm parameters are absorbed into the FC.
    Folding gamma into W and beta into a bias must give the same Y as
    normalising first (exact arithmetic; float64 here)."""
    rng = np.random.default_rng(seed)
    H = [rng.normal(0, sc, (M, d)) + rng.normal(0, 2.0, d) for sc in (1.0, 4.0, 16.0)]
    gam = [rng.normal(1, 0.1, d) for _ in range(3)]
    bet = [rng.normal(0, 0.05, d) for _ in range(3)]
    W = rng.normal(0, (3 * d) ** -0.5, (3 * d, d))
    bias = rng.normal(0, 0.01, d)
    for kind, eps in ((NORM_LN, 1e-5), (NORM_RMS, 1e-6), (NORM_NONE, 0.0)):
        b = bet if kind == NORM_LN else None
        Y = fuse_fn(H, kind, eps, gam, b, W, bias)
        Wf, u, c = fold_prepare(kind, gam, b, W, bias)
        Yf = fold_apply(H, kind, eps, Wf, u, c)
        if np.max(np.abs(Yf - Y)) > 1e-12 * max(1.0, np.max(np.abs(Y))):
            return False
    return True


# ---------------------------------------------------------------------------
# Post-norm hidden-state feedback: norm_fn(X, kind, eps, gamma, beta) -> [M, d]
# ---------------------------------------------------------------------------


def check_norm_output_torch(norm_fn, seed=17, d=96, M=7, tol=1e-12) -> bool:
    """Against torch's CPU float64 layer_norm / rms_norm (an independent
    library implementation), with and without gamma / beta; NONE returns x."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(seed)
    X = rng.normal(0, 6.0, (M, d)) + rng.normal(0, 2.0, d)
    g = rng.normal(1, 0.2, d)
    b = rng.normal(0, 0.1, d)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a))
    for gg, bb in ((g, b), (None, None), (g, None), (None, b)):
        ref = F.layer_norm(t(X), (d,), t(gg), t(bb), 1e-5).numpy()
        if np.max(np.abs(norm_fn(X, NORM_LN, 1e-5, gg, bb) - ref)) > tol * max(1.0, np.max(np.abs(ref))):
            return False
        ref = F.rms_norm(t(X), (d,), t(gg), 1e-6).numpy()
        # beta is not part of an RMSNorm: passing one must change nothing
        if np.max(np.abs(norm_fn(X, NORM_RMS, 1e-6, gg, bb) - ref)) > tol * max(1.0, np.max(np.abs(ref))):
            return False
    return bool(np.array_equal(norm_fn(X, NORM_NONE, 1e-5, g, b), X))


def check_norm_output_closed_forms(norm_fn, tol=1e-13) -> bool:
    """Rows whose statistics are known by hand.

    [1, 2, 3, 4]: mean 2.5, biased variance 1.25, mean square 7.5.
    A constant row c: LayerNorm gives beta exactly; RMSNorm c / sqrt(c^2 + eps).
    An alternating row +a, -a: mean 0, variance and mean square a^2.
    """
    g = np.array([1.0, 2.0, -0.5, 4.0])
    b = np.array([0.25, -1.0, 0.0, 3.0])
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    ok = np.allclose(norm_fn(x, NORM_LN, 0.0, None, None)[0], np.array([-1.5, -0.5, 0.5, 1.5]) / np.sqrt(1.25),
                     rtol=0, atol=tol)
    ok &= np.allclose(norm_fn(x, NORM_LN, 0.75, g, b)[0], np.array([-1.5, -0.5, 0.5, 1.5]) / np.sqrt(2.0) * g + b,
                      rtol=0, atol=tol)
    ok &= np.allclose(norm_fn(x, NORM_RMS, 0.5, g, None)[0], x[0] / np.sqrt(8.0) * g, rtol=0, atol=tol)
    c = np.full((2, 4), 3.0)
    c[1] = -0.125
    ok &= np.array_equal(norm_fn(c, NORM_LN, 1e-5, g, b), np.stack([b, b]))
    ok &= np.allclose(norm_fn(c, NORM_RMS, 1e-2, g, None), c / np.sqrt(c * c + 1e-2) * g, rtol=0, atol=tol)
    a = np.array([[5.0, -5.0, 5.0, -5.0]])
    want = a / np.sqrt(25.0 + 1e-3) * g
    ok &= np.allclose(norm_fn(a, NORM_LN, 1e-3, g, b), want + b, rtol=0, atol=tol)
    ok &= np.allclose(norm_fn(a, NORM_RMS, 1e-3, g, b), want, rtol=0, atol=tol)
    return bool(ok)


# ---------------------------------------------------------------------------
# Drafter-input concatenation: fn(tokens, embed_bits, fused_bits) -> (dst, bad)
# ---------------------------------------------------------------------------


def check_embed_concat_hand(fn) -> bool:
    """A table of 3 rows of width 2 and 4 tokens, the result written by hand."""
    embed = np.array([[1, 2], [3, 4], [5, 6]], dtype=np.uint16)
    fused = np.array([[10, 11], [12, 13], [14, 15], [16, 17]], dtype=np.uint16)
    tokens = np.array([2, 0, -1, 3], dtype=np.int32)
    want = np.array([[5, 6, 10, 11], [1, 2, 12, 13], [0, 0, 14, 15], [0, 0, 16, 17]], dtype=np.uint16)
    dst, bad = fn(tokens, embed, fused)
    return bool(np.array_equal(dst, want) and bad == 2)


def check_embed_concat_brute(fn, seed=31, M=9, d=5, vocab=4) -> bool:
    """Element-by-element loops over a small case with ids inside and outside
    the table."""
    rng = np.random.default_rng(seed)
    embed = rng.integers(1, 65535, size=(vocab, d)).astype(np.uint16)
    fused = rng.integers(1, 65535, size=(M, d)).astype(np.uint16)
    tokens = rng.integers(-2, vocab + 2, size=M).astype(np.int32)
    dst, bad = fn(tokens, embed, fused)
    nbad = 0
    for m in range(M):
        inside = 0 <= int(tokens[m]) < vocab
        nbad += 0 if inside else 1
        for j in range(d):
            if dst[m, j] != (embed[int(tokens[m]), j] if inside else 0):
                return False
            if dst[m, d + j] != fused[m, j]:
                return False
    return bad == nbad and dst.shape == (M, 2 * d)


# ---------------------------------------------------------------------------
# Verify / accept: fn(p, q, draft, u_acc, u_res) -> (n_accepted, next_token)
# ---------------------------------------------------------------------------


def check_verify_hand(fn) -> bool:
    """Worked by hand.  p_1 = (.5, .3, .2), q_1 = (.2, .5, .3): the draft 0 is
    kept when u < .4.  Residual (q_1 - p_1)+ = (0, .2, .1), total .3: u_res = .5
    aims at .15 -> token 1, u_res = .9 aims at .27 -> token 2.  A second draft
    (token 2, p_2 = (.6, .2, .2), q_2 = (.2, .2, .6): ratio 3, always kept) is
    never reached after a rejection at position 1.  All kept: the bonus from
    q_3 = (.1, .1, .8) with u_res = .5 aims at .5 -> token 2."""
    p = np.array([[[.5, .3, .2], [.6, .2, .2]]], dtype=np.float32)
    q = np.array([[[.2, .5, .3], [.2, .2, .6], [.1, .1, .8]]], dtype=np.float32)
    draft = np.array([[0, 2]])
    cases = [((.5, .1), .5, 0, 1), ((.5, .1), .9, 0, 2), ((.3, .1), .5, 2, 2), ((.3, .1), .05, 2, 0)]
    for ua, ur, n_want, t_want in cases:
        n, t = fn(p, q, draft, np.array([ua], dtype=np.float32), np.array([ur], dtype=np.float32))
        if int(n[0]) != n_want or int(t[0]) != t_want:
            return False
    return True


def check_verify_q_equals_p(fn, seed=41, B=64, N=4, V=50) -> bool:
    """With q = p every ratio is 1 > u, so all N drafts are kept and the
    bonus comes from q_{N+1} by inverse CDF (brute-force loop here)."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.ones(V), size=(B, N)).astype(np.float32)
    q = np.concatenate([p, rng.dirichlet(np.ones(V), size=(B, 1)).astype(np.float32)], axis=1)
    draft = rng.integers(0, V, size=(B, N))
    u_acc = rng.random((B, N), dtype=np.float32)
    u_res = rng.random(B, dtype=np.float32)
    n, t = fn(p, q, draft, u_acc, u_res)
    if not np.all(n == N):
        return False
    for b in range(B):
        w = q[b, N].astype(np.float64)
        target, run, pick = float(u_res[b]) * w.sum(), 0.0, V - 1
        for k in range(V):
            run += w[k]
            if run > target:
                pick = k
                break
        if int(t[b]) != pick:
            return False
    return True


def check_verify_leviathan(fn, seed=43, B=50000, V=8, alpha=0.05) -> bool:
    """The invariant the pages state: the emitted token follows q whatever p
    is.  50,000 seeded single-draft steps (draft ~ p); the first emitted token
    (the draft if kept, else the residual's) must pass, at the 95% critical
    value the lesson's exercise uses (section "연습문제", exercise 1):
    a chi-square goodness-of-fit test against q, and (section "직접 만들기",
    Step 5) a two-sample test against 50,000 tokens drawn from q directly by
    numpy's own sampler."""
    from scipy.stats import chi2

    rng = np.random.default_rng(seed)
    pr = rng.dirichlet(np.ones(V) * 0.7).astype(np.float32)
    qr = rng.dirichlet(np.ones(V) * 0.7).astype(np.float32)
    p = np.broadcast_to(pr, (B, 1, V))
    q = np.broadcast_to(qr, (B, 2, V))
    p64 = pr.astype(np.float64) / pr.astype(np.float64).sum()
    draft = rng.choice(V, size=B, p=p64)[:, None]
    n, t = fn(p, q, draft, rng.random((B, 1), dtype=np.float32), rng.random(B, dtype=np.float32))
    first = np.where(n == 1, draft[:, 0], t)
    if np.any(first < 0):
        return False
    counts = np.bincount(first, minlength=V).astype(np.float64)
    q64 = qr.astype(np.float64) / qr.astype(np.float64).sum()
    expect = q64 * B
    stat_fit = float(((counts - expect) ** 2 / expect).sum())
    direct = np.bincount(rng.choice(V, size=B, p=q64), minlength=V).astype(np.float64)
    used = (counts + direct) > 0
    stat_two = float(((counts[used] - direct[used]) ** 2 / (counts[used] + direct[used])).sum())
    crit = chi2.ppf(1 - alpha, V - 1)
    return stat_fit < crit and stat_two < chi2.ppf(1 - alpha, int(used.sum()) - 1)


def check_verify_zero_probability_drafts(fn) -> bool:
    """A draft the verifier gives zero probability is never kept, even when
    the drafter also gave it zero (q(d) = p(d) = 0); one with p(d) = 0 and
    q(d) > 0 is kept; an id outside the vocabulary is rejected.  After the
    rejection of a zero-zero draft with q = p the residual is all zero and the
    token comes from q itself (hand-worked: q = (.25, .75, 0), u_res = .5 aims
    at .5 -> token 1)."""
    p = np.array([[[.25, .75, 0.]]], dtype=np.float32)
    qsame = np.array([[[.25, .75, 0.], [1., 0., 0.]]], dtype=np.float32)
    qpos = np.array([[[.2, .5, .3], [0., 0., 1.]]], dtype=np.float32)
    ua = np.array([[.5]], dtype=np.float32)
    ur = np.array([.5], dtype=np.float32)
    n, t = fn(p, qsame, np.array([[2]]), ua, ur)
    if int(n[0]) != 0 or int(t[0]) != 1:
        return False
    n, t = fn(p, qpos, np.array([[2]]), ua, ur)          # kept, then the bonus from q_2 -> token 2
    if int(n[0]) != 1 or int(t[0]) != 2:
        return False
    for bad in (-1, 3, 1 << 20):                           # outside the vocabulary: rejected
        n, t = fn(p, qpos, np.array([[bad]]), ua, ur)
        # residual (q - p)+ = (0, 0, .3) -> token 2
        if int(n[0]) != 0 or int(t[0]) != 2:
            return False
    return True


def check_verify_invalid_rows(fn) -> bool:
    """No token (-1) when the weights sampled from are all zero, hold NaN or
    a value above 1, or u_res is outside [0, 1)."""
    p = np.array([[[.5, .5]]], dtype=np.float32)
    ok = np.array([[.9]], dtype=np.float32)                 # .9 * .5 < .5 is false: rejected
    keep = np.array([[.1]], dtype=np.float32)
    cases = [
        (np.array([[[.5, .5], [0., 0.]]], dtype=np.float32), keep, .5),          # bonus row all zero
        (np.array([[[.5, .5], [np.nan, .5]]], dtype=np.float32), keep, .5),      # bonus row with NaN
        (np.array([[[.5, .5], [2., .5]]], dtype=np.float32), keep, .5),          # bonus row above 1
        (np.array([[[np.nan, .5], [.5, .5]]], dtype=np.float32), ok, .5),        # residual with NaN
        (np.array([[[.5, .5], [.5, .5]]], dtype=np.float32), keep, 1.0),         # u_res = 1
        (np.array([[[.5, .5], [.5, .5]]], dtype=np.float32), keep, -0.25),       # u_res < 0
    ]
    for q, ua, ur in cases:
        _, t = fn(p, q, np.array([[0]]), ua, np.array([ur], dtype=np.float32))
        if int(t[0]) != -1:
            return False
    return True


def _inverse_cdf_fractions(w, u) -> int:
    """Direct definition with rational arithmetic: smallest t with
    w_0 + ... + w_t > u * total."""
    from fractions import Fraction
    ws = [Fraction(float(x)) for x in np.asarray(w, dtype=np.float32).tolist()]
    target = Fraction(float(np.float32(u))) * sum(ws, Fraction(0))
    run = Fraction(0)
    for t, x in enumerate(ws):
        run += x
        if run > target:
            return t
    return -1


def check_inverse_cdf_exact(fn_icdf, seed=47) -> bool:
    """The emitted token by inverse CDF, against the definition in rational
    arithmetic: seeded rows mixing ordinary, tiny (2^-100) and subnormal
    float32 weights and exact zeros; plus a hand case where running sums in
    float64 would pick another token: w = (.5, 2^-100, .5), u = .5 ->
    u * total = .5 + 2^-101, so the tiny weight's token 1 is the answer
    (float64 sums lose the 2^-100 and give 2)."""
    if fn_icdf(np.array([.5, 2.0 ** -100, .5], dtype=np.float32), np.float32(.5)) != 1:
        return False
    rng = np.random.default_rng(seed)
    for _ in range(200):
        V = int(rng.integers(1, 24))
        w = rng.random(V).astype(np.float32)
        kind = rng.integers(0, 4, size=V)
        w[kind == 1] = np.float32(2.0 ** -100) * (1 + np.float32(rng.random()))
        w[kind == 2] = np.float32(1e-42)                          # subnormal
        w[kind == 3] = 0
        u = np.float32(rng.random())
        if rng.random() < 0.2:                                   # u that lands on a boundary
            tot = sum(float(x) for x in w)
            u = np.float32(float(w[0]) / tot) if tot > 0 else u
        want = _inverse_cdf_fractions(w, u)
        if fn_icdf(w, u) != want:
            return False
    return True
