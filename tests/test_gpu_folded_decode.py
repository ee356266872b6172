"""The folded decode path (eagle31_fuse_folded, 1 <= M <= 128) against the
fp64 oracle through the C ABI, at every token-tile count and at widths that
change the split-K kernel's plan (columns per workgroup, waves, chunks per
state, ring depth), for all three norms; the decode-shaped workloads at every
token count; a 100-sigma DC offset through the fold; bitwise repeatability over
many calls at alternating token counts; the workspace-zeroing failure hook.

Tolerance: tests/parity.py (row-RMS-normalised max 2e-2, mean 4e-3).
"""

import numpy as np
import pytest

import oracle
import synth
from parity import DevInputs, assert_parity, bf16_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LN, RMS, NONE = 1, 2, 0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import eagle_draft_feature_amd  # noqa: F401
    yield
    torch.cuda.synchronize()


def e31():
    import eagle_draft_feature_amd as m
    return m


def note(msg):
    print(f"[case] {msg}", flush=True)


def oracle_out(inp, kind, eps):
    H = [oracle.decode_bf16(h) for h in inp.h]
    g = [oracle.decode_bf16(x) for x in inp.gamma]
    b = None if inp.beta is None else [oracle.decode_bf16(x) for x in inp.beta]
    bias = None if inp.bias is None else oracle.decode_bf16(inp.bias)
    return oracle.fuse(H, kind, eps, g, b, oracle.decode_bf16(inp.W), bias)


def folded_call(dv, kind, eps, prepared=None):
    wf, u, c = prepared if prepared is not None else e31().fold_prepare(kind, dv.gamma, dv.beta, dv.W, dv.bias)
    out = e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], kind, eps, wf, u, c)
    torch.cuda.synchronize()
    return out, (wf, u, c)


@pytest.mark.parametrize("d", [2048, 2560, 3072, 3584, 4096, 4608, 5120])
@pytest.mark.parametrize("M", [2, 3, 16, 17, 33, 64])
def test_folded_decode_parity(d, M):
    kind = (LN, RMS, NONE)[(d // 512 + M) % 3]
    eps = {LN: 1e-5, RMS: 1e-6, NONE: 0.0}[kind]
    note(f"folded decode d={d} M={M} kind={kind}")
    w = synth.gen.custom_workload(d, (M,), seed_tag=d * 13 + M)
    inp = synth.make_inputs(w, M)
    dv = DevInputs(inp)
    out, _ = folded_call(dv, kind, eps)
    assert_parity(bf16_to_f64(out), oracle_out(inp, kind, eps), f"folded d={d} M={M} kind={kind}")


@pytest.mark.parametrize("d", [512, 1280, 2048, 2304, 4096])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6])
def test_whole_k_kernel_few_tokens(d, M):
    """1 to 6 tokens at widths up to 4096, each workgroup walking the whole K
    for one 16-column block: at d = 2048 and 4096 with packed token blocks
    (16, 8, 4 or 2 k-steps per load; at d = 2048 one token takes two row
    slots), elsewhere with one or two tokens staged into LDS (chunk counts
    that do not fill a whole number of loads per thread wrap round) and more
    on the split kernels."""
    kind = (LN, RMS, NONE)[(d // 256 + M) % 3]
    eps = {LN: 1e-5, RMS: 1e-6, NONE: 0.0}[kind]
    note(f"whole-K decode d={d} M={M} kind={kind}")
    w = synth.gen.custom_workload(d, (M,), seed_tag=d * 7 + M)
    inp = synth.make_inputs(w, M)
    dv = DevInputs(inp)
    out, _ = folded_call(dv, kind, eps)
    assert_parity(bf16_to_f64(out), oracle_out(inp, kind, eps), f"whole-K d={d} M={M} kind={kind}")


@pytest.mark.parametrize("kind", [LN, RMS, NONE])
def test_folded_decode_every_norm_at_the_headline_shape(kind):
    note(f"folded decode d=4096 M=64 kind={kind}")
    inp = synth.make_inputs(2, 64)
    dv = DevInputs(inp)
    eps = {LN: 1e-5, RMS: 1e-6, NONE: 0.0}[kind]
    out, _ = folded_call(dv, kind, eps)
    assert_parity(bf16_to_f64(out), oracle_out(inp, kind, eps), f"folded headline kind={kind}")


def test_folded_decode_bitwise_over_many_calls():
    """Fifty-one calls back to back on one stream, at three token counts in
    turn (column split, and packed token blocks at three tokens): every output
    is bit-identical to the first of its size."""
    note("folded decode 51 repeats")
    inp = synth.make_inputs(2, 64)
    dv = DevInputs(inp)
    prepared = e31().fold_prepare(LN, dv.gamma, dv.beta, dv.W, dv.bias)
    refs = {}
    for M in (64, 9, 3):
        h = [x[:M] for x in dv.h]
        refs[M] = e31().fuse_folded(h[0], h[1], h[2], LN, 1e-5, *prepared)
    outs = []
    for i in range(51):
        M = (64, 9, 3)[i % 3]
        h = [x[:M] for x in dv.h]
        outs.append((M, e31().fuse_folded(h[0], h[1], h[2], LN, 1e-5, *prepared)))
    torch.cuda.synchronize()
    for M, o in outs:
        assert torch.equal(o.view(torch.int16), refs[M].view(torch.int16)), f"repeat differs at M={M}"
    assert_parity(bf16_to_f64(refs[9]), oracle_out(inp.rows(9), LN, 1e-5), "folded M=9")
    assert_parity(bf16_to_f64(refs[3]), oracle_out(inp.rows(3), LN, 1e-5), "folded M=3")


@pytest.mark.parametrize("d,M,kind", [(3584, 64, LN), (3584, 17, NONE), (5120, 33, RMS), (8192, 2, LN),
                                      (4096, 64, RMS)])
def test_folded_decode_stats_fallback_same_bits_every_chunking(d, M, kind):
    """The statistics readers' fallback (recompute the rows), forced from the
    host, gives the same bits as the normal path at chunkings with 4, 6, 7 and
    8 K chunks (d=3584: chunks that cross a state boundary, so a chunk's part
    applies two states' statistics) and 1, 2, 3, 4 token tiles; both match
    the oracle."""
    eps = {LN: 1e-5, RMS: 1e-6, NONE: 0.0}[kind]
    note(f"stats fallback d={d} M={M} kind={kind}")
    w = synth.gen.custom_workload(d, (M,), seed_tag=d * 7 + M)
    inp = synth.make_inputs(w, M)
    dv = DevInputs(inp)
    normal, prepared = folded_call(dv, kind, eps)
    e31().debug_stats_recompute(True)
    try:
        forced, _ = folded_call(dv, kind, eps, prepared)
    finally:
        e31().debug_stats_recompute(False)
    assert torch.equal(normal.view(torch.int16), forced.view(torch.int16)), "fallback differs"
    assert_parity(bf16_to_f64(forced), oracle_out(inp, kind, eps), f"fallback d={d} M={M} kind={kind}")


@pytest.mark.parametrize("d,M,kind", [(4096, 65, LN), (4096, 128, LN), (5120, 128, RMS), (5120, 96, LN),
                                      (3584, 113, NONE), (8192, 100, RMS), (3072, 80, LN), (4608, 127, LN)])
def test_folded_decode_up_to_eight_token_tiles(d, M, kind):
    """65 to 128 tokens (5 to 8 token tiles) take the column-split decode
    kernel where its plan exists: parity with the oracle at widths with 4, 6,
    7 and 8 K chunks, and the forced statistics fallback gives the same bits."""
    eps = {LN: 1e-5, RMS: 1e-6, NONE: 0.0}[kind]
    note(f"folded decode 5-8 tiles d={d} M={M} kind={kind}")
    w = synth.gen.custom_workload(d, (M,), seed_tag=d * 3 + M)
    inp = synth.make_inputs(w, M)
    dv = DevInputs(inp)
    out, prepared = folded_call(dv, kind, eps)
    assert_parity(bf16_to_f64(out), oracle_out(inp, kind, eps), f"folded d={d} M={M} kind={kind}")
    if kind != NONE:
        e31().debug_stats_recompute(True)
        try:
            forced, _ = folded_call(dv, kind, eps, prepared)
        finally:
            e31().debug_stats_recompute(False)
        assert torch.equal(out.view(torch.int16), forced.view(torch.int16)), "fallback differs"


def test_folded_decode_stats_fallback_cost_is_bounded():
    """If the workgroups that publish the statistics do not run (another
    stream holding the CUs), a reader waits at most ~200 us and then computes
    the rows itself.  The fallback, forced from the host, is timed here at the
    decode batch: its cost plus the wait bound is what such a call can lose."""
    note("stats fallback timing d=4096 M=64")
    inp = synth.make_inputs(2, 64)
    dv = DevInputs(inp)
    prepared = e31().fold_prepare(LN, dv.gamma, dv.beta, dv.W, dv.bias)
    out = torch.empty((64, dv.d), dtype=torch.bfloat16, device="cuda")

    def per_call_us(n=20):
        for _ in range(3):
            e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], LN, 1e-5, *prepared, out=out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], LN, 1e-5, *prepared, out=out)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    normal = per_call_us()
    e31().debug_stats_recompute(True)
    try:
        forced = per_call_us()
    finally:
        e31().debug_stats_recompute(False)
    print(f"[timing] folded decode d=4096 M=64: {normal:.1f} us per call, {forced:.1f} us with the statistics "
          f"fallback in every reader", flush=True)
    assert forced < 2000.0, f"the fallback path took {forced:.0f} us per call"


@pytest.mark.parametrize("M", [4, 64])
def test_folded_decode_dc_offset(M):
    """A shared offset of 100 sigma on h_high through the folded path: the
    statistics' shifted sums and the fold's h.W' - mu.u cancellation hold."""
    note(f"folded decode dc offset M={M}")
    w = synth.gen.custom_workload(4096, (M,), seed_tag=71)
    inp = synth.make_inputs(w, M, extra_offset=(0.0, 0.0, 1600.0))
    dv = DevInputs(inp)
    out, _ = folded_call(dv, LN, 1e-5)
    assert_parity(bf16_to_f64(out), oracle_out(inp, LN, 1e-5), f"folded dc offset M={M}")


def test_workspace_zeroing_failure_keeps_no_buffer():
    """A library-owned workspace whose counter zeroing fails (forced by the
    test hook) is not kept: the call reports the HIP failure, and the next
    call on that stream allocates and zeroes a fresh buffer and is correct."""
    note("workspace zero hook")
    inp = synth.make_inputs(2, 64)
    dv = DevInputs(inp)
    prepared = e31().fold_prepare(LN, dv.gamma, dv.beta, dv.W, dv.bias)
    s = torch.cuda.Stream()
    e31().debug_fail_workspace_zero(True)
    try:
        with torch.cuda.stream(s):
            with pytest.raises(e31().Eagle31Error):
                e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], LN, 1e-5, *prepared)
    finally:
        e31().debug_fail_workspace_zero(False)
    with torch.cuda.stream(s):
        out = e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], LN, 1e-5, *prepared)
    torch.cuda.synchronize()
    assert_parity(bf16_to_f64(out), oracle_out(inp, LN, 1e-5), "after zero hook")
