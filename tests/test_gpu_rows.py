"""eagle31_fuse_rows / eagle31_fuse_folded_rows through the C ABI: the hidden
states read where they are (strided views, an index list of source rows), the
output written into a wider buffer.

Every case is checked two ways on the same seeded inputs:
* bit for bit against the dense entry point (eagle31_fuse / _folded) run on
  a contiguous copy of the gathered rows: the same kernels with only the
  addressing changed must give the same bits;
* against the fp64 oracle applied to the gathered rows (tests/parity.py
  bars; all rows of decode batches, sampled rows of prefill batches).
Layouts: the three states as column blocks of one [n, 3d + 64] buffer, and
three separate buffers with different row paddings (ld = d, d + 64, d + 24).
Index lists with repeats and any order, ragged M (1 to 3000: the one-token,
split-K decode, split-K prefill and plain prefill kernels), indices outside
the buffer (zero rows), output rows 2d apart in the drafter-input buffer
whose other half must stay untouched, and that buffer completed by
eagle31_embed_concat without a fused argument, bit-exact against the
concatenation oracle.
"""

import numpy as np
import pytest

import oracle
import synth
from parity import DevInputs, assert_parity, bf16_to_f64, sample_rows, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LN, RMS, NONE = 1, 2, 0
SENTINEL = 0x1234  # bf16 bits left in the half of the output buffer that must stay untouched


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


def note(msg):
    print(f"[case] {msg}", flush=True)


_cache = {}


def inputs(cfg, n_src):
    key = (cfg, n_src)
    if key not in _cache:
        if len(_cache) > 2:
            _cache.clear()
        inp = synth.make_inputs(cfg, n_src)
        _cache[key] = (inp, DevInputs(inp))
    return _cache[key]


def place(dv: DevInputs, layout: str):
    """The device states in the given layout: returns three [n, d] views."""
    n, d = dv.M, dv.d
    if layout == "interleaved":
        buf = torch.zeros((n, 3 * d + 64), dtype=torch.bfloat16, device="cuda")
        for s in range(3):
            buf[:, s * d:(s + 1) * d] = dv.h[s]
        return [buf[:, s * d:(s + 1) * d] for s in range(3)]
    views = []
    for s, pad in enumerate((0, 64, 24)):
        b = torch.zeros((n, d + pad), dtype=torch.bfloat16, device="cuda")
        b[:, :d] = dv.h[s]
        views.append(b[:, :d])
    return views


def index_list(n_src, M, seed, bad=()):
    """M source rows: repeats and any order; positions in `bad` get indices
    outside [0, n_src)."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, n_src, size=M).astype(np.int64)
    if M > 3:
        idx[: M // 3] = idx[: M // 3][::-1]  # a reversed run
        idx[-1] = idx[0]                     # a repeat
    for k, pos in enumerate(bad):
        idx[pos] = (-1, n_src, 2 ** 31 - 1, -(2 ** 31))[k % 4]
    return idx.astype(np.int32)


def out_buffer(M, d):
    dst = torch.full((M, 2 * d), 0, dtype=torch.int16, device="cuda")
    dst.fill_(SENTINEL)
    return dst.view(torch.bfloat16)


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dense_reference(dv, kind, eps, folded, idx, wfc=None):
    """The dense entry point on a contiguous copy of the gathered rows (indices
    outside the buffer replaced by row 0; those rows are not compared)."""
    valid = (idx >= 0) & (idx < dv.M)
    sel = torch.from_numpy(np.where(valid, idx, 0).astype(np.int64)).to("cuda")
    g = [torch.index_select(h, 0, sel).contiguous() for h in dv.h]
    if folded:
        wf, u, c = wfc
        y = e31().fuse_folded(g[0], g[1], g[2], kind, eps, wf, u, c)
    else:
        y = e31().fuse(g[0], g[1], g[2], kind, eps, dv.gamma, dv.beta, dv.W, dv.bias)
    torch.cuda.synchronize()
    return y, valid


def oracle_gathered(inp, kind, eps, rows_src):
    H = [oracle.decode_bf16(h[rows_src]) for h in inp.h]
    g = [oracle.decode_bf16(x) for x in inp.gamma]
    b = [oracle.decode_bf16(x) for x in inp.beta] if inp.beta is not None else None
    bias = oracle.decode_bf16(inp.bias) if inp.bias is not None else None
    return oracle.fuse(H, kind, eps, g, b, oracle.decode_bf16(inp.W), bias)


def run_case(cfg, n_src, M, kind, eps, folded, layout, seed, bad=(), oracle_rows=None):
    inp, dv = inputs(cfg, n_src)
    d = dv.d
    note(f"rows cfg{cfg} n_src={n_src} M={M} kind={kind} folded={folded} layout={layout} bad={len(bad)}")
    views = place(dv, layout)
    idx = index_list(n_src, M, seed, bad)
    idx_t = torch.from_numpy(idx).to("cuda")
    dst = out_buffer(M, d)
    wfc = e31().fold_prepare(kind, dv.gamma, dv.beta, dv.W, dv.bias) if folded else None
    if folded:
        wf, u, c = wfc
        e31().fuse_folded_rows(views[0], views[1], views[2], kind, eps, wf, u, c, row_index=idx_t, out=dst[:, d:])
    else:
        e31().fuse_rows(views[0], views[1], views[2], kind, eps, dv.gamma, dv.beta, dv.W, dv.bias, row_index=idx_t,
                        out=dst[:, d:])
    torch.cuda.synchronize()
    got = bits(dst)
    # the other half of every output row is untouched
    assert (got[:, :d] == SENTINEL).all(), "the left half of the output buffer was written"
    ref, valid = dense_reference(dv, kind, eps, folded, idx, wfc)
    want = bits(ref)
    right = got[:, d:]
    assert (right[~valid] == 0).all(), "rows of indices outside the buffer must be zeros"
    mism = np.nonzero((right[valid] != want[valid]).any(axis=1))[0]
    print(f"[rows] bit-exact vs dense on {int(valid.sum())} rows: {len(mism)} rows differ", flush=True)
    assert len(mism) == 0, f"rows differ from the dense path: {np.nonzero(valid)[0][mism[:8]]}"
    rows = oracle_rows(M) if oracle_rows is not None else np.zeros(0, dtype=np.int64)
    rows = rows[valid[rows]]
    if len(rows):
        Y = oracle_gathered(inp, kind, eps, idx[rows])
        G = bf16_to_f64(dst[:, d:][torch.from_numpy(rows).to("cuda")])
        assert_parity(G, Y, f"rows cfg{cfg} M={M} vs oracle")
    return dst, idx, wfc


ALL = lambda M: np.arange(M)  # noqa: E731


@pytest.mark.parametrize("M,layout", [(1, "interleaved"), (3, "padded"), (4, "interleaved"), (7, "padded"),
                                      (64, "interleaved"), (64, "padded"), (100, "interleaved"), (128, "padded")])
def test_folded_decode_rows(M, layout):
    """Up to 64 tokens the decode kernels (one or two tokens staged whole
    into each workgroup's LDS); 100 and 128 take the column-split kernel's 7 and 8
    token tiles (source rows of tokens 64 .. from the second per-lane
    register)."""
    run_case(2, 160, M, LN, 1e-5, True, layout, seed=M, oracle_rows=ALL)


@pytest.mark.parametrize("M,layout", [(1, "padded"), (16, "interleaved"), (61, "padded")])
def test_stored_decode_rows(M, layout):
    run_case(2, 100, M, LN, 1e-5, False, layout, seed=100 + M, oracle_rows=ALL)


@pytest.mark.parametrize("cfg,n_src,M,kind,eps,folded,layout", [
    (2, 500, 300, LN, 1e-5, True, "interleaved"),     # split-K prefill
    (2, 3500, 3000, LN, 1e-5, True, "padded"),        # plain prefill, ragged tile
    (3, 300, 256, RMS, 1e-6, True, "padded"),         # RMS, no beta / bias
    (3, 64, 37, RMS, 1e-6, True, "interleaved"),      # RMS decode
    (1, 400, 200, NONE, 0.0, True, "padded"),         # no norm
    (2, 500, 300, LN, 1e-5, False, "padded"),         # stored W: per-call fold + prefill
])
def test_prefill_and_norm_kinds_rows(cfg, n_src, M, kind, eps, folded, layout):
    run_case(cfg, n_src, M, kind, eps, folded, layout, seed=cfg * 7 + M,
             oracle_rows=lambda m: sample_rows(m, k=40, seed=3))


@pytest.mark.parametrize("M,folded", [(1, True), (1, False), (40, True), (40, False), (97, True), (300, True)])
def test_indices_outside_the_buffer_give_zero_rows(M, folded):
    bad = (0,) if M == 1 else (0, M // 2, M - 1, 5)
    run_case(2, 120, M, LN, 1e-5, folded, "padded", seed=900 + M, bad=bad, oracle_rows=ALL if M < 64 else None)


def test_no_index_list_strided_views():
    """Without an index list token m reads row m of each (strided) view."""
    inp, dv = inputs(2, 64)
    d = dv.d
    note("rows: strided views, no index")
    views = place(dv, "interleaved")
    wf, u, c = e31().fold_prepare(LN, dv.gamma, dv.beta, dv.W, dv.bias)
    dst = out_buffer(64, d)
    e31().fuse_folded_rows(views[0], views[1], views[2], LN, 1e-5, wf, u, c, out=dst[:, d:])
    ref = e31().fuse_folded(dv.h[0], dv.h[1], dv.h[2], LN, 1e-5, wf, u, c)
    torch.cuda.synchronize()
    got = bits(dst)
    assert (got[:, :d] == SENTINEL).all()
    assert np.array_equal(got[:, d:], bits(ref))


@pytest.mark.parametrize("M", [1, 64, 300])
def test_drafter_input_buffer_without_a_copy(M):
    """The fused feature written into the right half of the drafter-input
    buffer by the fusion itself, the left half by eagle31_embed_concat with no
    fused argument: the buffer equals the concatenation oracle bit for bit."""
    dst, idx, wfc = run_case(2, 400, M, LN, 1e-5, True, "interleaved", seed=M + 5)
    _, dv = inputs(2, 400)
    d = dv.d
    tokens, embed_bits, _ = synth.make_embed_inputs(M, d, 1000, seed=M, n_bad=2 if M > 1 else 0)
    e31().embed_concat(torch.from_numpy(tokens).to("cuda"), to_dev(embed_bits), None, out=dst)
    torch.cuda.synchronize()
    fused_bits = bits(dense_reference(dv, LN, 1e-5, True, idx, wfc)[0])
    want, _ = oracle.embed_concat(tokens, embed_bits, fused_bits)
    got = bits(dst)
    mism = np.nonzero((got != want).any(axis=1))[0]
    print(f"[rows] drafter-input buffer M={M}: {len(mism)} rows differ from the oracle", flush=True)
    assert len(mism) == 0
