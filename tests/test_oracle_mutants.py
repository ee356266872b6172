"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each mutant is a copy of the oracle's fusion with one plausible slip: a
dropped term, a wrong sign or index, a wrong estimator, a swapped operand.
None of these is imported by anything else; they exist to show the pins
have teeth.
"""

import numpy as np
import pytest

import oracle
import oracle_pins as pins

NONE, LN, RMS = 0, 1, 2


def _make(norm_fn, order=(0, 1, 2), use_bias=True, fc=None):
    def fuse(H, kind, eps, gam, bet, W, bias):
        parts = []
        for s in order:
            g = None if gam is None else gam[s]
            b = None if bet is None else bet[s]
            parts.append(norm_fn(np.asarray(H[s], float), kind, eps, g, b))
        X = np.concatenate(parts, axis=1)
        Y = X @ W if fc is None else fc(X, W)
        if use_bias and bias is not None:
            Y = Y + bias
        return Y
    return fuse


def _ln_family(var_fn=None, eps_outside=False, affine=True, beta=True, rms_mean=False, gamma_first=False):
    def norm(X, kind, eps, g, b):
        d = X.shape[1]
        g = np.ones(d) if g is None else g
        b = np.zeros(d) if b is None else b
        if kind == NONE:
            return X.copy()
        if kind == LN or (kind == RMS and rms_mean):
            mu = X.mean(1)
            v = ((X - mu[:, None]) ** 2).mean(1) if var_fn is None else var_fn(X, mu)
            r = 1 / (np.sqrt(v) + eps) if eps_outside else 1 / np.sqrt(v + eps)
            if gamma_first:
                return (X * g - mu[:, None]) * r[:, None] + (b if beta else 0)
            out = (X - mu[:, None]) * r[:, None]
            if affine:
                out = out * g
            if beta and kind == LN:
                out = out + b
            return out
        ms = (X * X).mean(1)
        r = 1 / (np.sqrt(ms) + eps) if eps_outside else 1 / np.sqrt(ms + eps)
        out = X * r[:, None]
        return out * g if affine else out
    return norm


MUTANTS = {
    "variance_without_centering": _make(_ln_family(var_fn=lambda X, mu: (X * X).mean(1))),
    "unbiased_variance": _make(_ln_family(var_fn=lambda X, mu: ((X - mu[:, None]) ** 2).sum(1) / (X.shape[1] - 1))),
    "eps_outside_sqrt": _make(_ln_family(eps_outside=True)),
    "gamma_dropped": _make(_ln_family(affine=False)),
    "beta_dropped": _make(_ln_family(beta=False)),
    "rms_subtracts_mean": _make(_ln_family(rms_mean=True)),
    "gamma_before_centering": _make(_ln_family(gamma_first=True)),
    "segments_low_high_swapped": _make(_ln_family(), order=(2, 1, 0)),
    "bias_dropped": _make(_ln_family(), use_bias=False),
    "fc_sign_flipped": _make(_ln_family(), fc=lambda X, W: -(X @ W)),
    "fc_rows_reversed_within_segment": _make(
        _ln_family(), fc=lambda X, W: X @ np.concatenate(
            [W[s * W.shape[1]:(s + 1) * W.shape[1]][::-1] for s in range(3)])),
}


def _all_pins(fuse_fn):
    rng = np.random.default_rng(1)
    d, M = 24, 6
    H = [rng.normal(0, sc, (M, d)) + rng.normal(0, 0.5, d) for sc in (1.0, 4.0, 16.0)]
    gam = [rng.normal(1, 0.1, d) for _ in range(3)]
    W = rng.normal(0, (3 * d) ** -0.5, (3 * d, d))
    bias = rng.normal(0, 0.01, d)
    return {
        "hand": pins.check_hand_example(fuse_fn),
        "moments": pins.check_moments(fuse_fn, H),
        "scale": pins.check_scale_invariance(fuse_fn, H, gam, W, bias),
        "scale_eps": pins.check_scale_invariance_eps(fuse_fn, H, gam, W, bias),
        "brute": pins.check_brute_force(fuse_fn),
        "torch": pins.check_torch_library(fuse_fn),
        "none": pins.check_none_is_eagle3(fuse_fn),
        "order": pins.check_segment_order(fuse_fn),
        "rows": pins.check_row_independence(fuse_fn),
    }


def test_pins_pass_on_oracle():
    res = _all_pins(oracle.fuse)
    assert all(res.values()), res


def test_reference_copy_of_oracle_passes():
    """The unmutated family used to build mutants passes every pin, so a
    mutant's failure is due to its one slip."""
    res = _all_pins(_make(_ln_family()))
    assert all(res.values()), res


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    res = _all_pins(MUTANTS[name])
    assert not all(res.values()), f"mutant {name} passed every pin: {res}"


# --- post-norm feedback: planted slips in the row norm -----------------------


def _postnorm_mutant(slip):
    def norm_fn(X, kind, eps, g, b):
        X = np.asarray(X, float)
        d = X.shape[1]
        g = np.ones(d) if g is None else np.asarray(g, float)
        b = np.zeros(d) if b is None else np.asarray(b, float)
        if kind == NONE:
            return X.copy()
        if kind == LN:
            mu = X.mean(axis=1, keepdims=True)
            var = ((X - mu) ** 2).sum(axis=1, keepdims=True) / (d - 1 if slip == "unbiased" else d)
            r = 1.0 / (np.sqrt(var) + eps) if slip == "eps_outside" else 1.0 / np.sqrt(var + eps)
            return (X - mu) * r * g + (0.0 if slip == "no_beta" else b)
        mu = X.mean(axis=1, keepdims=True) if slip == "rms_centres" else 0.0
        r = 1.0 / np.sqrt(((X - mu) ** 2).mean(axis=1, keepdims=True) + eps)
        out = (X - mu) * r
        return out if slip == "no_gamma" else out * g
    return norm_fn


@pytest.mark.parametrize("slip", ["unbiased", "eps_outside", "no_beta", "rms_centres", "no_gamma"])
def test_postnorm_mutants_fail_a_pin(slip):
    fn = _postnorm_mutant(slip)
    assert not (pins.check_norm_output_torch(fn) and pins.check_norm_output_closed_forms(fn))


def test_postnorm_mutant_harness_is_faithful():
    """The unmutated copy passes every pin (so a failure above is the slip's)."""
    fn = _postnorm_mutant(None)
    assert pins.check_norm_output_torch(fn) and pins.check_norm_output_closed_forms(fn)


# --- drafter-input concatenation: planted slips ---------------------------------


def _embedcat_mutant(slip):
    def fn(tokens, embed, fused):
        tokens = np.asarray(tokens, dtype=np.int64)
        vocab, d = embed.shape
        ok = (tokens >= 0) & (tokens < vocab)
        if slip == "clamp_ids":
            left = embed[np.clip(tokens, 0, vocab - 1)]
        else:
            t = tokens + 1 if slip == "off_by_one" else tokens
            ok2 = (t >= 0) & (t < vocab)
            left = np.zeros((len(tokens), d), dtype=np.uint16)
            left[ok2] = embed[t[ok2]]
        parts = [fused, left] if slip == "swapped" else [left, fused]
        bad = int(np.count_nonzero(~ok)) + (1 if slip == "count" else 0)
        return np.concatenate(parts, axis=1), bad
    return fn


@pytest.mark.parametrize("slip", ["clamp_ids", "off_by_one", "swapped", "count"])
def test_embedcat_mutants_fail_a_pin(slip):
    fn = _embedcat_mutant(slip)
    assert not (pins.check_embed_concat_hand(fn) and pins.check_embed_concat_brute(fn))


def test_embedcat_mutant_harness_is_faithful():
    fn = _embedcat_mutant(None)
    assert pins.check_embed_concat_hand(fn) and pins.check_embed_concat_brute(fn)


# --- verify / accept: planted slips ---------------------------------------------


def _verify_mutant(slip):
    import oracle.verify64 as v

    def icdf(w, u):
        if slip == "float64_cdf":
            w = np.asarray(w, dtype=np.float32)
            if not (0 <= float(u) < 1) or not np.all((w >= 0) & (w <= 1)) or not np.any(w > 0):
                return -1
            c = np.cumsum(w.astype(np.float64))
            return int(np.searchsorted(c, float(u) * c[-1], side="right"))
        return v.inverse_cdf(w, u)

    def fn(p, q, draft, u_acc, u_res):
        p = np.asarray(p, dtype=np.float32)
        q = np.asarray(q, dtype=np.float32)
        B, N, V = p.shape
        n_acc = np.zeros(B, dtype=np.int32)
        nxt = np.zeros(B, dtype=np.int32)
        for b in range(B):
            j, rejected = N, False
            for i in range(N):
                t = int(draft[b, i])
                inside = 0 <= t < V or slip == "wrap_ids"
                pd = p[b, i, t % V] if inside else np.float32(0)
                qd = q[b, i, t % V] if inside else np.float32(0)
                if slip == "inverted_ratio":
                    keep = np.float32(u_acc[b, i]) * qd < pd
                elif slip == "keep_zero_p":
                    keep = pd <= 0 or np.float32(u_acc[b, i]) * pd < qd
                else:
                    keep = np.float32(u_acc[b, i]) * pd < qd
                if not keep:
                    if not rejected:
                        j, rejected = i, True
                    if slip != "no_stop":
                        break
                elif slip == "no_stop" and rejected:
                    j += 1
            n_acc[b] = j
            if j < N:
                if slip == "flipped_residual":
                    w = np.maximum(p[b, j] - q[b, j], 0)
                elif slip == "unclipped":
                    w = np.abs(q[b, j] - p[b, j])
                else:
                    w = np.maximum(q[b, j] - p[b, j], 0)
                if np.all((w >= 0) & (w <= 1)) and not np.any(w > 0):
                    w = q[b, j]
            else:
                w = q[b, N - 1 if slip == "bonus_row" else N]
            nxt[b] = icdf(w, u_res[b])
        return n_acc, nxt
    return fn, icdf


VERIFY_SLIPS = ["inverted_ratio", "flipped_residual", "unclipped", "bonus_row", "no_stop", "keep_zero_p",
                "wrap_ids", "float64_cdf"]


def _verify_pins_pass(fn, icdf):
    return (pins.check_verify_hand(fn) and pins.check_verify_q_equals_p(fn) and pins.check_verify_leviathan(fn)
            and pins.check_verify_zero_probability_drafts(fn) and pins.check_verify_invalid_rows(fn)
            and pins.check_inverse_cdf_exact(icdf))


@pytest.mark.parametrize("slip", VERIFY_SLIPS)
def test_verify_mutants_fail_a_pin(slip):
    assert not _verify_pins_pass(*_verify_mutant(slip))


def test_verify_mutant_harness_is_faithful():
    assert _verify_pins_pass(*_verify_mutant(None))
