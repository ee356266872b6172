"""Every row of the full-size workloads against the fp64 oracle: the
long-context prefill (d=7168, M=32768, LayerNorm, outlier channels) and the
chunked prefill (d=8192, M=512/2048/4093/4096, LayerNorm and RMSNorm), through
both entry points (eagle31_fuse on the stored weight, eagle31_fuse_folded on
the prepared one); scale invariance at the long-context size.

The oracle runs in row chunks (the step is row independent, so the chunks
are exact pieces of the full result); each workload's oracle is computed once
per module.  Tolerance: tests/parity.py, assert_parity_full (mean bar as
written; max bar element by element with the bf16 output grid accounted for).
"""

import numpy as np
import pytest

import oracle
import synth
from parity import DevInputs, assert_parity_full, bf16_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LN, RMS = 1, 2


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


def oracle_chunked(inp, kind, eps, chunk=4096):
    """Oracle over all rows, chunk by chunk (exact: rows are independent)."""
    g = [oracle.decode_bf16(x) for x in inp.gamma]
    b = None if (inp.beta is None or kind != LN) else [oracle.decode_bf16(x) for x in inp.beta]
    W = oracle.decode_bf16(inp.W)
    bias = None if inp.bias is None else oracle.decode_bf16(inp.bias)
    Y = np.empty((inp.M, inp.d), dtype=np.float64)
    for r0 in range(0, inp.M, chunk):
        H = [oracle.decode_bf16(h[r0:r0 + chunk]) for h in inp.h]
        Y[r0:r0 + chunk] = oracle.fuse(H, kind, eps, g, b, W, bias)
    return Y


def run(dv, kind, eps, folded, M=None, h=None):
    M = dv.M if M is None else M
    h = [x[:M] for x in dv.h] if h is None else h
    if folded:
        wf, u, c = e31().fold_prepare(kind, dv.gamma, dv.beta, dv.W, dv.bias)
        out = e31().fuse_folded(h[0], h[1], h[2], kind, eps, wf, u, c)
        del wf
    else:
        out = e31().fuse(h[0], h[1], h[2], kind, eps, dv.gamma, dv.beta, dv.W, dv.bias)
    torch.cuda.synchronize()
    G = bf16_to_f64(out)
    del out
    return G


# ------------------------------------------------- long-context prefill (cfg 4)
@pytest.fixture(scope="module")
def long_prefill():
    note("long-context prefill: generating d=7168 M=32768 and the oracle over every row")
    inp = synth.make_inputs(4)
    Y = oracle_chunked(inp, LN, 1e-5)
    dv = DevInputs(inp)
    yield inp, dv, Y
    del dv
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("folded", [False, True])
def test_long_prefill_every_row(long_prefill, folded):
    inp, dv, Y = long_prefill
    note(f"long prefill d=7168 M=32768 LN folded={folded}: every row")
    G = run(dv, LN, 1e-5, folded)
    assert_parity_full(G, Y, f"long prefill folded={folded}")


@pytest.mark.timeout(900)
def test_long_prefill_scale_invariance(long_prefill):
    """LayerNorm output does not change when a state is scaled (with beta too:
    beta is added after the normalisation), so scaling h_high by 4 and h_low by
    1/4 (exact in bfloat16) must still match the same oracle; the deviation
    from the unscaled GPU output is reported."""
    inp, dv, Y = long_prefill
    note("long prefill scale invariance: h_low x 1/4, h_high x 4")
    h = [dv.h[0] * 0.25, dv.h[1], dv.h[2] * 4.0]
    G = run(dv, LN, 1e-5, False, h=h)
    del h
    assert_parity_full(G, Y, "long prefill scaled")
    G0 = run(dv, LN, 1e-5, False)
    rms = np.sqrt(np.mean(Y * Y, axis=1, keepdims=True))
    print(f"[scale] long prefill: max |G(scaled) - G| / RMS = {float(np.max(np.abs(G - G0) / rms)):.3e}")


# --------------------------------------------------- chunked prefill (cfg 5)
@pytest.fixture(scope="module")
def chunked():
    note("chunked prefill: generating d=8192 M=4096 and the oracle (LN, RMS) over every row")
    inp = synth.make_inputs(5, 4096)
    Ys = {LN: oracle_chunked(inp, LN, 1e-5), RMS: oracle_chunked(inp, RMS, 1e-6)}
    dv = DevInputs(inp)
    yield inp, dv, Ys
    del dv
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("folded", [False, True])
@pytest.mark.parametrize("kind,eps", [(LN, 1e-5), (RMS, 1e-6)])
@pytest.mark.parametrize("M", [512, 2048, 4093, 4096])
def test_chunked_prefill_every_row(chunked, M, kind, eps, folded):
    inp, dv, Ys = chunked
    note(f"chunked prefill d=8192 M={M} kind={kind} folded={folded}: every row")
    G = run(dv, kind, eps, folded, M=M)
    assert_parity_full(G, Ys[kind][:M], f"chunked M={M} kind={kind} folded={folded}")
