"""HIP path (through the C ABI) against the fp64 oracle, on the same seeded
bfloat16 inputs.  Needs an MI355X: every test here is marked gpu.

Tolerance: tests/parity.py (row-RMS-normalised max 2e-2, mean 4e-3).
The full-size prefill workloads are checked on every row in
tests/test_gpu_fullsize.py; the d=4160 pipeline-restart case here checks
sampled rows plus its whole ragged last tile.
"""

import numpy as np
import pytest

import oracle
import synth
from parity import DevInputs, assert_parity, bf16_to_f64, sample_rows, to_dev, unpack_folded

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LN, RMS, NONE = 1, 2, 0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import eagle_draft_feature_amd  # noqa: F401  (fails loudly if the library is missing)
    yield
    torch.cuda.synchronize()


def e31():
    import eagle_draft_feature_amd as m
    return m


_cache = {}


def inputs(cfg, M=None, **kw):
    key = (cfg if isinstance(cfg, int) else cfg.name, M, tuple(sorted(kw.items())))
    if key not in _cache:
        if len(_cache) > 3:
            _cache.clear()
        _cache[key] = synth.make_inputs(cfg, M, **kw)
    return _cache[key]


def run_fuse(dv: DevInputs, kind, eps, use_beta=True, use_gamma=True, use_bias=True, M=None):
    M = dv.M if M is None else M
    h = [x[:M] for x in dv.h]
    out = e31().fuse(h[0], h[1], h[2], kind, eps, dv.gamma if use_gamma else None,
                     dv.beta if use_beta else None, dv.W, dv.bias if use_bias else None)
    torch.cuda.synchronize()
    return bf16_to_f64(out)


def oracle_rows(inp, kind, eps, rows=None, use_beta=True, use_gamma=True, use_bias=True):
    H = [oracle.decode_bf16(h if rows is None else h[rows]) for h in inp.h]
    g = [oracle.decode_bf16(x) for x in inp.gamma] if use_gamma else None
    b = [oracle.decode_bf16(x) for x in inp.beta] if (use_beta and inp.beta is not None) else None
    bias = oracle.decode_bf16(inp.bias) if (use_bias and inp.bias is not None) else None
    return oracle.fuse(H, kind, eps, g, b, oracle.decode_bf16(inp.W), bias)


def note(msg):
    print(f"[case] {msg}", flush=True)


# ----------------------------------------------------------------- row stats
@pytest.mark.parametrize("cfg,M,kind,eps", [(1, 64, LN, 1e-5), (2, 64, LN, 1e-5), (3, 256, RMS, 1e-6),
                                            (5, 512, LN, 1e-5), (5, 512, RMS, 1e-6)])
def test_row_stats(cfg, M, kind, eps):
    note(f"row_stats cfg{cfg} M={M} kind={kind}")
    inp = synth.make_inputs(cfg, M, with_weights=False)
    h = [to_dev(x) for x in inp.h]
    mu, rstd = e31().row_stats(h[0], h[1], h[2], kind, eps)
    torch.cuda.synchronize()
    mu, rstd = mu.cpu().numpy().astype(np.float64), rstd.cpu().numpy().astype(np.float64)
    for s in range(3):
        X = oracle.decode_bf16(inp.h[s])
        mo, ro = oracle.row_stats(X, kind, eps)
        sd = X.std(axis=1)
        assert np.max(np.abs(mu[s] - mo) / sd) < 1e-5, s
        assert np.max(np.abs(rstd[s] / ro - 1)) < 1e-5, s


# ------------------------------------------------------------ small configs
@pytest.mark.parametrize("M", [64])
def test_cfg1_tiny_layernorm(M):
    note("cfg1 d=512 M=64 LN")
    inp = inputs(1)
    dv = DevInputs(inp)
    G = run_fuse(dv, LN, 1e-5)
    assert_parity(G, oracle_rows(inp, LN, 1e-5), "cfg1")


@pytest.mark.parametrize("M", [1, 4, 8, 16, 64])
def test_cfg2_decode_layernorm(M):
    note(f"cfg2 d=4096 M={M} LN")
    inp = inputs(2, 64)
    dv = DevInputs(inp)
    G = run_fuse(dv, LN, 1e-5, M=M)
    assert_parity(G, oracle_rows(inp.rows(M), LN, 1e-5), f"cfg2 M={M}")


@pytest.mark.parametrize("M", [64, 128, 256])
def test_cfg3_tree_rmsnorm(M):
    note(f"cfg3 d=5120 M={M} RMS")
    inp = inputs(3, 256)
    dv = DevInputs(inp)
    G = run_fuse(dv, RMS, 1e-6, M=M)
    assert_parity(G, oracle_rows(inp.rows(M), RMS, 1e-6), f"cfg3 M={M}")


@pytest.mark.parametrize("folded", [False, True])
def test_prefill_state_restart_ragged(folded):
    """Prefill without split-K at a width whose state length is not a whole
    number of pipeline cycles (d = 4160: 130 sub-tiles of 32 per state), so
    the pipeline restarts at every state; M = 3100 leaves a ragged last
    M-tile.  Sampled rows plus every row of the ragged tile."""
    note(f"prefill restart d=4160 M=3100 folded={folded}")
    d, M = 4160, 3100
    w = synth.gen.custom_workload(d, (M,), seed_tag=4160)
    inp = synth.make_inputs(w, M)
    dv = DevInputs(inp)
    if folded:
        wf, u, c = e31().fold_prepare(LN, dv.gamma, dv.beta, dv.W, dv.bias)
        G = bf16_to_f64(e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], LN, 1e-5, wf, u, c))
    else:
        G = run_fuse(dv, LN, 1e-5)
    rows = np.unique(np.concatenate([sample_rows(M, 24, seed=41), np.arange(3072, M)]))
    assert_parity(G[rows], oracle_rows(inp, LN, 1e-5, rows=rows), f"prefill restart folded={folded}")
    del dv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d,M,kind", [(7168, 512, LN), (4096, 700, RMS), (8192, 300, LN)])
def test_prefill_four_chunks_across_states(d, M, kind):
    """43 to 64 output tiles: K split into four equal chunks that cross the
    state boundaries, each storing one partial per state part (56, 48 and 64
    tiles; M = 700 and 300 leave ragged last M-tiles).  Both entry points,
    every row against the oracle, and the same bits on a second call."""
    eps = {LN: 1e-5, RMS: 1e-6}[kind]
    note(f"prefill four chunks d={d} M={M} kind={kind}")
    w = synth.gen.custom_workload(d, (M,), seed_tag=d + M)
    inp = synth.make_inputs(w, M)
    dv = DevInputs(inp)
    Y = oracle_rows(inp, kind, eps)
    wf, u, c = e31().fold_prepare(kind, dv.gamma, dv.beta, dv.W, dv.bias)
    F1 = e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], kind, eps, wf, u, c)
    F2 = e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], kind, eps, wf, u, c)
    torch.cuda.synchronize()
    assert torch.equal(F1.view(torch.int16), F2.view(torch.int16)), "second call differs"
    assert_parity(bf16_to_f64(F1), Y, f"four chunks folded d={d} M={M}")
    assert_parity(run_fuse(dv, kind, eps), Y, f"four chunks stored W d={d} M={M}")
    del dv, wf, u, c, F1, F2
    torch.cuda.empty_cache()


# ------------------------------------------------------------ the fold path
@pytest.mark.parametrize("cfg,kind,eps", [(1, LN, 1e-5), (3, RMS, 1e-6), (1, NONE, 0.0)])
def test_fold_prepare_exact_weight_and_vectors(cfg, kind, eps):
    """W' = bf16_rne(gamma * W) has one correct answer (the product of two
    bfloat16 values is exact): bit-exact.  u and c are float32 sums."""
    note(f"fold_prepare cfg{cfg} kind={kind}")
    inp = inputs(cfg, 64 if cfg == 1 else 256)
    dv = DevInputs(inp)
    wf, u, c = e31().fold_prepare(kind, dv.gamma, dv.beta, dv.W, dv.bias)
    torch.cuda.synchronize()
    W = oracle.decode_bf16(inp.W)
    g = [oracle.decode_bf16(x) for x in inp.gamma]
    b = None if inp.beta is None else [oracle.decode_bf16(x) for x in inp.beta]
    bias = None if inp.bias is None else oracle.decode_bf16(inp.bias)
    Wf, uo, co = oracle.fold_prepare(kind, g, b, W, bias, round_w=oracle.round_bf16_rne)
    got = unpack_folded(bf16_to_f64(wf), inp.d)
    assert np.array_equal(got, Wf), f"W' mismatch in {np.sum(got != Wf)} elements"
    uo_scale = np.abs(Wf).sum() / Wf.shape[1] / 3
    assert np.max(np.abs(u.cpu().numpy() - uo)) <= 1e-5 * max(uo_scale, 1.0)
    assert np.max(np.abs(c.cpu().numpy() - co)) <= 1e-5 * max(np.abs(co).max(), 1e-3) + 1e-6


@pytest.mark.parametrize("cfg,M,kind,eps", [(1, 64, LN, 1e-5), (2, 1, LN, 1e-5), (2, 4, LN, 1e-5), (2, 8, LN, 1e-5),
                                            (2, 16, LN, 1e-5), (2, 32, LN, 1e-5), (2, 64, LN, 1e-5),
                                            (3, 64, RMS, 1e-6), (3, 128, RMS, 1e-6), (3, 256, RMS, 1e-6)])
def test_fuse_folded_parity(cfg, M, kind, eps):
    note(f"fuse_folded cfg{cfg} M={M} kind={kind}")
    inp = inputs(cfg, synth.CONFIGS[cfg].max_M if cfg != 2 else 64)
    dv = DevInputs(inp)
    wf, u, c = e31().fold_prepare(kind, dv.gamma, dv.beta, dv.W, dv.bias)
    h = [x[:M] for x in dv.h]
    out = e31().fuse_folded(h[0], h[1], h[2], kind, eps, wf, u, c)
    torch.cuda.synchronize()
    G = bf16_to_f64(out)
    assert_parity(G, oracle_rows(inp.rows(M), kind, eps), f"folded cfg{cfg} M={M}")


@pytest.mark.parametrize("cfg,M,kind,eps", [(2, 1, LN, 1e-5), (2, 64, LN, 1e-5), (3, 64, RMS, 1e-6),
                                            (1, 17, LN, 1e-5), (1, 64, NONE, 0.0)])
def test_folded_stats_recompute_path_same_bits(cfg, M, kind, eps):
    """The folded decode kernel hands each token's statistics between
    workgroups; a reader that does not find them computes the rows itself.
    Forced from the host, that fallback gives the same bits as the normal
    path, and both match the oracle."""
    note(f"stats recompute path cfg{cfg} M={M} kind={kind}")
    inp = inputs(cfg, synth.CONFIGS[cfg].max_M if cfg != 2 else 64)
    dv = DevInputs(inp)
    wf, u, c = e31().fold_prepare(kind, dv.gamma, dv.beta, dv.W, dv.bias)
    h = [x[:M] for x in dv.h]
    normal = e31().fuse_folded(h[0], h[1], h[2], kind, eps, wf, u, c)
    torch.cuda.synchronize()
    e31().debug_stats_recompute(True)
    try:
        forced = e31().fuse_folded(h[0], h[1], h[2], kind, eps, wf, u, c)
        torch.cuda.synchronize()
    finally:
        e31().debug_stats_recompute(False)
    assert torch.equal(normal.view(torch.int16), forced.view(torch.int16)), "fallback statistics differ"
    again = e31().fuse_folded(h[0], h[1], h[2], kind, eps, wf, u, c)
    torch.cuda.synchronize()
    assert torch.equal(normal.view(torch.int16), again.view(torch.int16))
    assert_parity(bf16_to_f64(forced), oracle_rows(inp.rows(M), kind, eps), f"recompute cfg{cfg} M={M}")


# ------------------------------------------------ properties and edge cases
@pytest.mark.parametrize("cfg,M,kind", [(1, 64, LN), (2, 16, LN), (3, 64, RMS), (5, 512, LN)])
def test_gpu_scale_invariance(cfg, M, kind):
    """beta = 0: scaling one state by a power of two (exact in bfloat16)
    leaves the output unchanged up to rounding, on the GPU too."""
    note(f"scale invariance cfg{cfg} M={M}")
    eps = 1e-5 if kind == LN else 1e-6
    inp = inputs(cfg, M if cfg != 2 else 64)
    dv = DevInputs(inp)
    base = run_fuse(dv, kind, eps, use_beta=False, M=M)
    Y = oracle_rows(inp.rows(M), kind, eps, use_beta=False)
    assert_parity(base, Y, f"scale base cfg{cfg}")
    worst = 0.0
    for s in range(3):
        for cscale in (0.25, 4.0, 16.0):
            h = [x[:M] for x in dv.h]
            h[s] = (h[s].float() * cscale).to(torch.bfloat16)
            out = e31().fuse(h[0], h[1], h[2], kind, eps, dv.gamma, None, dv.W, dv.bias)
            torch.cuda.synchronize()
            Gc = bf16_to_f64(out)
            mx, _ = assert_parity(Gc, Y, f"scaled s={s} c={cscale}")
            worst = max(worst, mx)
    print(f"[scale] cfg{cfg}: worst max deviation vs oracle {worst:.3e}")


def test_none_mode_is_eagle3():
    note("NONE mode cfg1 / cfg2 M=8 / cfg5 M=512")
    for cfg, M in ((1, 64), (2, 8), (5, 512)):
        inp = inputs(cfg, M if cfg != 2 else 64)
        dv = DevInputs(inp)
        G = run_fuse(dv, NONE, 0.0, M=M)
        assert_parity(G, oracle_rows(inp.rows(M), NONE, 0.0), f"none cfg{cfg} M={M}")


@pytest.mark.parametrize("cfg,M", [(2, 64), (5, 2048), (3, 128)])
def test_bitwise_determinism(cfg, M):
    note(f"determinism cfg{cfg} M={M}")
    inp = inputs(cfg, M if cfg != 2 else 64)
    dv = DevInputs(inp)
    kind, eps = synth.CONFIGS[cfg].norms[0]
    a = run_fuse(dv, kind, eps, M=M)
    b = run_fuse(dv, kind, eps, M=M)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("M", [16, 64, 600])
def test_dc_offset_stress(M):
    """A shared offset of 100 sigma on h_high: a variance formed as
    E[x^2] - mean^2 in float32 would lose most of its digits."""
    note(f"dc offset M={M}")
    w = synth.gen.custom_workload(1024, (M,), seed_tag=7)
    inp = synth.make_inputs(w, M, extra_offset=(0.0, 0.0, 1600.0))
    dv = DevInputs(inp)
    G = run_fuse(dv, LN, 1e-5)
    assert_parity(G, oracle_rows(inp, LN, 1e-5), f"dc offset M={M}")


@pytest.mark.parametrize("d,M,kind", [(64, 1, LN), (64, 3, RMS), (192, 65, LN), (320, 70, RMS), (128, 257, LN),
                                      (384, 300, NONE), (256, 1000, LN), (4160, 5, LN)])
def test_edge_shapes(d, M, kind):
    """Minimum width, widths that are not multiples of 128 or 256 (column
    tails), ragged token counts on both paths, the decode/prefill boundary."""
    note(f"edge d={d} M={M} kind={kind}")
    w = synth.gen.custom_workload(d, (M,), seed_tag=d * 7 + M)
    inp = synth.make_inputs(w, M)
    dv = DevInputs(inp)
    eps = 1e-5
    G = run_fuse(dv, kind, eps)
    assert_parity(G, oracle_rows(inp, kind, eps), f"edge d={d} M={M}")


@pytest.mark.parametrize("d,M,kind", [(64, 1, LN), (64, 3, RMS), (192, 17, LN), (320, 33, RMS), (512, 64, NONE),
                                      (1024, 40, LN), (4160, 5, LN), (5120, 64, RMS)])
def test_folded_edge_shapes(d, M, kind):
    """The folded decode kernel at widths that change its plan (waves per
    workgroup, chunks per state, ring depth) and ragged token counts."""
    note(f"folded edge d={d} M={M} kind={kind}")
    w = synth.gen.custom_workload(d, (M,), seed_tag=d * 11 + M)
    inp = synth.make_inputs(w, M)
    dv = DevInputs(inp)
    eps = 1e-5
    wf, u, c = e31().fold_prepare(kind, dv.gamma, dv.beta, dv.W, dv.bias)
    out = e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], kind, eps, wf, u, c)
    torch.cuda.synchronize()
    assert_parity(bf16_to_f64(out), oracle_rows(inp, kind, eps), f"folded edge d={d} M={M}")


def test_two_streams_use_their_own_workspaces():
    """Calls in flight on two streams at once each use the library-owned
    workspace of their own stream: interleaved calls with no synchronisation
    between them give the same bits as the same calls run one at a time.
    Stream 1 runs the folded decode kernel (d=4096, M=64); stream 2 alternates
    the folded decode kernel at d=512 and the split-K prefill path (d=512,
    M=300, stored weight)."""
    note("two streams")
    inpA = inputs(2, 64)
    inpB = inputs(1)
    w = synth.gen.custom_workload(512, (300,), seed_tag=77)
    inpC = synth.make_inputs(w, 300)
    dA, dB, dC = DevInputs(inpA), DevInputs(inpB), DevInputs(inpC)
    fA = e31().fold_prepare(LN, dA.gamma, dA.beta, dA.W, dA.bias)
    fB = e31().fold_prepare(LN, dB.gamma, dB.beta, dB.W, dB.bias)

    def callA():
        return e31().fuse_folded(dA.h[0], dA.h[1], dA.h[2], LN, 1e-5, *fA)

    def callB():
        return e31().fuse_folded(dB.h[0], dB.h[1], dB.h[2], LN, 1e-5, *fB)

    def callC():
        return e31().fuse(dC.h[0], dC.h[1], dC.h[2], LN, 1e-5, dC.gamma, dC.beta, dC.W, dC.bias)

    refA, refB, refC = callA(), callB(), callC()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(6):
        with torch.cuda.stream(s1):
            outs.append(("A", callA()))
        with torch.cuda.stream(s2):
            outs.append(("B", callB()) if i % 2 == 0 else ("C", callC()))
    torch.cuda.synchronize()
    ref = {"A": refA, "B": refB, "C": refC}
    for name, o in outs:
        assert torch.equal(o.view(torch.int16), ref[name].view(torch.int16)), f"stream result {name} differs"
    assert_parity(bf16_to_f64(refC), oracle_rows(inpC, LN, 1e-5), "two streams, prefill path")


@pytest.mark.parametrize("d", [512, 1024, 2048, 3072, 4096, 5120, 8192])
@pytest.mark.parametrize("kind", [LN, RMS, NONE])
def test_one_token_kernel_widths(d, kind):
    """A single token at widths that change the one-token plan, for every
    norm: packed token blocks at d = 2048, 4096 and 8192 (two rounds of
    workgroups), the LDS-staged whole-K kernel at 512, 1024 and 3072, the
    split-K kernel at 5120."""
    note(f"one token d={d} kind={kind}")
    w = synth.gen.custom_workload(d, (1,), seed_tag=d + 7 * kind)
    inp = synth.make_inputs(w, 1)
    dv = DevInputs(inp)
    eps = 1e-5 if kind == LN else (1e-6 if kind == RMS else 0.0)
    wf, u, c = e31().fold_prepare(kind, dv.gamma, dv.beta, dv.W, dv.bias)
    out = e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], kind, eps, wf, u, c)
    again = e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], kind, eps, wf, u, c)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    assert_parity(bf16_to_f64(out), oracle_rows(inp, kind, eps), f"one token d={d} kind={kind}")
    # the stored-weight entry point (its own one-token kernel), with and
    # without the optional parameters
    Y = oracle_rows(inp, kind, eps)
    G = run_fuse(dv, kind, eps)
    assert_parity(G, Y, f"one token stored W d={d} kind={kind}")
    assert np.array_equal(G, run_fuse(dv, kind, eps))
    if kind != NONE:
        G0 = run_fuse(dv, kind, eps, use_gamma=False, use_beta=False, use_bias=False)
        Y0 = oracle_rows(inp, kind, eps, use_gamma=False, use_beta=False, use_bias=False)
        assert_parity(G0, Y0, f"one token stored W, no parameters, d={d} kind={kind}")


def test_optional_parameters_absent():
    """gamma = None means 1, beta = None means 0, bias = None means none."""
    note("optional params")
    inp = inputs(1)
    dv = DevInputs(inp)
    for ug, ub, ubias in ((False, False, False), (True, False, True), (False, True, False)):
        G = run_fuse(dv, LN, 1e-5, use_gamma=ug, use_beta=ub, use_bias=ubias)
        Y = oracle_rows(inp, LN, 1e-5, use_gamma=ug, use_beta=ub, use_bias=ubias)
        assert_parity(G, Y, f"params g={ug} b={ub} bias={ubias}")


@pytest.mark.parametrize("cfg,M", [(2, 16), (5, 512)])
def test_caller_workspace_matches_owned(cfg, M):
    note(f"fuse_ws cfg{cfg} M={M}")
    inp = inputs(cfg, M if cfg != 2 else 64)
    dv = DevInputs(inp)
    kind, eps = synth.CONFIGS[cfg].norms[0]
    h = [x[:M] for x in dv.h]
    n = e31().workspace_size(M, inp.d, kind)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    e31().workspace_init(ws)
    a = e31().fuse_ws(h[0], h[1], h[2], kind, eps, dv.gamma, dv.beta, dv.W, dv.bias, ws)
    b = e31().fuse(h[0], h[1], h[2], kind, eps, dv.gamma, dv.beta, dv.W, dv.bias)
    a2 = e31().fuse_ws(h[0], h[1], h[2], kind, eps, dv.gamma, dv.beta, dv.W, dv.bias, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, a2)


def test_alternating_paths_share_workspace():
    """Decode and prefill calls in turn on one stream reuse the same
    library workspace; the counters each path uses start at zero."""
    note("alternating decode/prefill")
    inp = inputs(5, 512)
    dv = DevInputs(inp)
    ref_small = run_fuse(dv, LN, 1e-5, M=32)
    ref_big = run_fuse(dv, LN, 1e-5, M=512)
    for _ in range(2):
        assert np.array_equal(run_fuse(dv, LN, 1e-5, M=512), ref_big)
        assert np.array_equal(run_fuse(dv, LN, 1e-5, M=32), ref_small)
    assert_parity(ref_small, oracle_rows(inp.rows(32), LN, 1e-5), "alt small")
