"""eagle31_norm_output (post-norm hidden-state feedback) through the C ABI
against the fp64 oracle, on seeded bfloat16 rows.  Needs an MI355X.

Tolerance, from the arithmetic: the device computes the statistics and the
affine map in float32 and rounds the result once to bfloat16 (nearest even),
so per element |G - Y| <= 2^-8 |Y| (half a bfloat16 ulp) plus the float32
error of the statistics, about 2^-24 of the row's scale; the bound below
allows 1e-5 of the row's largest |Y| for it.  The fusion tests' mean bar
(4e-3 of the row RMS) holds as well; their max bar (2e-2 of the row RMS) does
not fit here: the output is one rounding of the normalised row itself, and in
the heavy-tailed rows an element near 28 sigma is off by up to 2^-8 * 28, about
0.11 of the row RMS, while still within half an ulp.  NONE is a copy and must
be bit-exact.
"""

import numpy as np
import pytest

import oracle
import synth
from parity import assert_parity, bf16_to_f64, sample_rows, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LN, RMS, NONE = 1, 2, 0
NAMES = {LN: "layernorm", RMS: "rmsnorm", NONE: "none"}


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


def rows_of(d, M, seed_tag, state=2):
    """Seeded drafter-output stand-in: one hidden state of the workload
    generator (heavy-tailed rows, per-column offsets) with its gamma / beta."""
    inp = synth.make_inputs(synth.gen.custom_workload(d, (M,), seed_tag=seed_tag), M, with_weights=False)
    return inp.h[state], inp.gamma[state], inp.beta[state]


def assert_elementwise(G, Y, what):
    assert G.shape == Y.shape
    assert np.all(np.isfinite(G)), what
    bound = 2.0 ** -8 * np.abs(Y) * (1 + 1e-5) + 1e-5 * np.max(np.abs(Y), axis=1, keepdims=True)
    bad = np.abs(G - Y) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond half a bf16 ulp, first at {np.argwhere(bad)[0]}"
    assert_parity(G, Y, what, max_tol=np.inf)


def run(x_bits, kind, eps, g_bits, b_bits, out=None):
    x = to_dev(x_bits)
    g = None if g_bits is None else to_dev(g_bits)
    b = None if b_bits is None else to_dev(b_bits)
    o = e31().norm_output(x, NAMES[kind], eps, g, b, out=out)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("d", [64, 1088, 4096, 7168, 8192])
@pytest.mark.parametrize("M", [1, 37])
@pytest.mark.parametrize("kind", [LN, RMS])
@pytest.mark.parametrize("params", [True, False])
def test_norm_output_parity(d, M, kind, params):
    """Widths from one 16-byte piece per lane (64) through a ragged piece
    count (1088: 136 pieces, 8 lanes in the last round) to the largest (8192)."""
    print(f"[case] norm_output d={d} M={M} kind={kind} params={params}", flush=True)
    x, g, b = rows_of(d, M, seed_tag=1000 + d + M)
    eps = 1e-5 if kind == LN else 1e-6
    gb, bb = (g, b) if params else (None, None)
    G = bf16_to_f64(run(x, kind, eps, gb, bb))
    Y = oracle.norm_output_bits(x, kind, eps, gb, bb if kind == LN else None)
    assert_elementwise(G, Y, f"norm_output d={d} M={M} kind={kind} params={params}")


@pytest.mark.parametrize("d", [64, 1088, 8192])
def test_norm_output_none_is_a_copy(d):
    print(f"[case] norm_output none d={d}", flush=True)
    x, g, b = rows_of(d, 19, seed_tag=7)
    o = run(x, NONE, 0.0, g, b)
    assert np.array_equal(o.view(torch.int16).cpu().numpy().view(np.uint16), x)


@pytest.mark.parametrize("kind", [LN, RMS])
@pytest.mark.parametrize("d", [1088, 4096])
def test_norm_output_in_place_same_bits(kind, d):
    """out == x: each row is read whole before it is written, so the result
    equals the out-of-place call bit for bit."""
    print(f"[case] norm_output in place d={d} kind={kind}", flush=True)
    x, g, b = rows_of(d, 300, seed_tag=11)
    ref = run(x, kind, 1e-5, g, b).view(torch.int16).cpu().numpy()
    xt = to_dev(x)
    o = e31().norm_output(xt, NAMES[kind], 1e-5, to_dev(g), to_dev(b), out=xt)
    torch.cuda.synchronize()
    assert o.data_ptr() == xt.data_ptr()
    assert np.array_equal(xt.view(torch.int16).cpu().numpy(), ref)


def test_norm_output_decode_shape_exhaustive_and_repeatable():
    """The decode batch's shape (M=64, d=4096, LayerNorm with gamma and beta):
    every element against the oracle, and the same bits on a second call."""
    print("[case] norm_output decode d=4096 M=64", flush=True)
    inp = synth.make_inputs(2, M=64, with_weights=False)
    x, g, b = inp.h[1], inp.gamma[1], inp.beta[1]
    o1 = run(x, LN, 1e-5, g, b)
    o2 = run(x, LN, 1e-5, g, b)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert_elementwise(bf16_to_f64(o1), oracle.norm_output_bits(x, LN, 1e-5, g, b), "norm_output decode M=64")


def test_norm_output_prefill_shape_sampled():
    """The prefill batch's shape (M=32768, d=7168, LayerNorm) in the launch
    the bench times (grid-stride rows, 512 workgroups): sampled rows against
    the oracle row by row (rows are independent)."""
    print("[case] norm_output prefill d=7168 M=32768 (sampled rows)", flush=True)
    inp = synth.make_inputs(4, M=32768, with_weights=False)
    x, g, b = inp.h[2], inp.gamma[2], inp.beta[2]
    G = bf16_to_f64(run(x, LN, 1e-5, g, b))
    rows = sample_rows(32768, k=96, seed=3)
    Y = oracle.norm_output_bits(x[rows], LN, 1e-5, g, b)
    assert_elementwise(G[rows], Y, "norm_output prefill sampled")


@pytest.mark.parametrize("kind", [LN, RMS])
def test_norm_output_grid_stride_ragged(kind):
    """More rows than the grid has waves (512 workgroups x 8 waves), at a
    ragged width (1088: the last round of pieces has 8 lanes): every wave
    takes two rows, some of its lanes re-read and re-write a clamped piece.
    Every row against the oracle."""
    print(f"[case] norm_output grid stride d=1088 M=4500 kind={kind}", flush=True)
    x, g, b = rows_of(1088, 4500, seed_tag=23)
    eps = 1e-5 if kind == LN else 1e-6
    G = bf16_to_f64(run(x, kind, eps, g, b))
    Y = oracle.norm_output_bits(x, kind, eps, g, b if kind == LN else None)
    assert_elementwise(G, Y, f"norm_output grid stride kind={kind}")
