"""The fp64 oracle against what the pages and the mathematics fix (CPU only).

Each check lives in tests/oracle_pins.py and takes the fusion function under
test, so tests/test_oracle_mutants.py can show that plausible slips fail them.
"""

import numpy as np
import pytest

import oracle
import oracle_pins as pins
import synth


def _small_H(d=24, M=6, seed=1):
    rng = np.random.default_rng(seed)
    H = [rng.normal(0, sc, (M, d)) + rng.normal(0, 0.5, d) for sc in (1.0, 4.0, 16.0)]
    gam = [rng.normal(1, 0.1, d) for _ in range(3)]
    W = rng.normal(0, (3 * d) ** -0.5, (3 * d, d))
    bias = rng.normal(0, 0.01, d)
    return H, gam, W, bias


def test_hand_example_closed_forms():
    assert pins.check_hand_example(oracle.fuse)


def test_moments_small():
    H, _, _, _ = _small_H()
    assert pins.check_moments(oracle.fuse, H)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_moments_on_workload_inputs(cfg):
    """Moments of every state of every workload's generated inputs (a row
    sample at full width; gamma = 1, beta = 0).  LN at eps = 0: mean 0 and
    variance 1 to 1e-9; at eps > 0: variance v / (v + eps).  RMS: mean square
    1 (eps = 0) or ms / (ms + eps)."""
    inp = synth.make_inputs(cfg, M=min(64, synth.CONFIGS[cfg].max_M), with_weights=False)
    d = inp.d
    H = [oracle.decode_bf16(h) for h in inp.h]
    ones, zeros = np.ones(d), np.zeros(d)
    for s in range(3):
        v = np.var(H[s], axis=1)
        ms = np.mean(H[s] ** 2, axis=1)
        for eps in (0.0, 1e-5):
            n = oracle.normalize(H[s], oracle.NORM_LN, eps, ones, zeros)
            assert np.max(np.abs(n.mean(axis=1))) <= 1e-9
            target = 1.0 if eps == 0.0 else v / (v + eps)
            assert np.max(np.abs(n.var(axis=1) - target)) <= 1e-9
            r = oracle.normalize(H[s], oracle.NORM_RMS, eps, ones, None)
            target = 1.0 if eps == 0.0 else ms / (ms + eps)
            assert np.max(np.abs(np.mean(r ** 2, axis=1) - target)) <= 1e-9


def test_scale_invariance_exact_at_eps0():
    H, gam, W, bias = _small_H()
    assert pins.check_scale_invariance(oracle.fuse, H, gam, W, bias)


def test_scale_invariance_eps_closed_form():
    H, gam, W, bias = _small_H()
    assert pins.check_scale_invariance_eps(oracle.fuse, H, gam, W, bias)


def test_brute_force_d4_M2():
    assert pins.check_brute_force(oracle.fuse)


def test_torch_library_cross_check():
    assert pins.check_torch_library(oracle.fuse)


def test_none_is_eagle3_fusion():
    assert pins.check_none_is_eagle3(oracle.fuse)


def test_segment_order_low_mid_high():
    assert pins.check_segment_order(oracle.fuse)


def test_row_independence():
    assert pins.check_row_independence(oracle.fuse)


def test_fold_identity():
    assert pins.check_fold_identity(oracle.fuse, oracle.fold_prepare, oracle.fold_apply)


def test_fuse_bits_matches_decoded_fuse_and_rows():
    """fuse_bits is fuse on the decoded bit patterns; a row subset gives the
    same rows as the full call (row independence used by sampled parity)."""
    inp = synth.make_inputs(1)
    Y = oracle.fuse_bits(inp, oracle.NORM_LN, 1e-5)
    rows = np.array([0, 5, 63, 17])
    Ys = oracle.fuse_bits(inp, oracle.NORM_LN, 1e-5, rows=rows)
    assert np.array_equal(Ys, Y[rows])
    H = [oracle.decode_bf16(h) for h in inp.h]
    assert H[0].dtype == np.float64 and H[0].shape == (64, 512)


def test_decode_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x3C00], dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 0.0, -0.0, 3.3895313892515355e38, 2.0 ** -7]
    assert np.array_equal(oracle.decode_bf16(bits), np.array(want))


def test_round_bf16_rne_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -30, 255.5, 256.5])
    want = np.array([1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7, 256.0, 256.0])
    assert np.array_equal(oracle.round_bf16_rne(x), want)


def test_generator_prefix_rule_and_determinism():
    a = synth.make_inputs(5, M=16, with_weights=False)
    b = synth.make_inputs(5, M=13, with_weights=False)
    for s in range(3):
        assert np.array_equal(a.h[s][:13], b.h[s])
    c = synth.make_inputs(5, M=16, with_weights=False)
    assert all(np.array_equal(a.h[s], c.h[s]) for s in range(3))


def test_generator_distribution_recipe():
    """Sanity of the synthetic recipe: state scales grow low < mid < high,
    outlier channels of the long-prefill workload are ~20x."""
    inp = synth.make_inputs(4, M=256, with_weights=False)
    H = [oracle.decode_bf16(h) for h in inp.h]
    stds = [np.median(np.std(h, axis=0)) for h in H]
    assert stds[0] < stds[1] < stds[2]
    colstd = np.std(H[2], axis=0)
    top = np.sort(colstd)[-8:]
    assert np.all(top > 10 * np.median(colstd))


def test_norm_output_torch_library_cross_check():
    assert pins.check_norm_output_torch(oracle.norm_output)


def test_norm_output_closed_forms():
    assert pins.check_norm_output_closed_forms(oracle.norm_output)


def test_norm_output_bits_decodes_like_fuse_inputs():
    """norm_output_bits on generated bf16 rows equals norm_output on the
    exactly decoded values (row 0 of the low state and its parameters)."""
    inp = synth.make_inputs(1, M=8, with_weights=False)
    got = oracle.norm_output_bits(inp.h[0], oracle.NORM_LN, 1e-5, inp.gamma[0], inp.beta[0])
    want = oracle.norm_output(oracle.decode_bf16(inp.h[0]), oracle.NORM_LN, 1e-5, oracle.decode_bf16(inp.gamma[0]),
                              oracle.decode_bf16(inp.beta[0]))
    assert np.array_equal(got, want)


def test_embed_concat_hand_example():
    assert pins.check_embed_concat_hand(oracle.embed_concat)


def test_embed_concat_brute_force():
    assert pins.check_embed_concat_brute(oracle.embed_concat)


def test_verify_hand_example():
    import oracle.verify64 as v
    assert pins.check_verify_hand(v.verify_accept)


def test_verify_q_equals_p_keeps_everything():
    import oracle.verify64 as v
    assert pins.check_verify_q_equals_p(v.verify_accept)


def test_verify_emitted_token_follows_q():
    import oracle.verify64 as v
    assert pins.check_verify_leviathan(v.verify_accept)


def test_verify_zero_probability_drafts():
    import oracle.verify64 as v
    assert pins.check_verify_zero_probability_drafts(v.verify_accept)


def test_verify_invalid_rows_give_no_token():
    import oracle.verify64 as v
    assert pins.check_verify_invalid_rows(v.verify_accept)


def test_inverse_cdf_exact_against_fractions():
    import oracle.verify64 as v
    assert pins.check_inverse_cdf_exact(v.inverse_cdf)
