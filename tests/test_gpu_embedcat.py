"""eagle31_embed_concat (the drafter's input row: previous token's embedding,
then the fused feature) through the C ABI against the oracle.  Byte work:
every output bit must match, and so must the count of token ids outside the
table.  Needs an MI355X."""

import numpy as np
import pytest

import oracle
import synth
from parity import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import eagle_draft_feature_amd  # noqa: F401  (fails loudly if the library is missing)
    yield
    torch.cuda.synchronize()


def run(tokens, embed, fused, count=True):
    import eagle_draft_feature_amd as e31
    tok = torch.from_numpy(tokens).to("cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda") if count else None
    out = e31.embed_concat(tok, to_dev(embed), to_dev(fused), bad_count=bad)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return bits, (None if bad is None else int(bad.item()))


@pytest.mark.parametrize("M,d,vocab,n_bad", [
    (1, 64, 7, 0),        # one piece per lane
    (1, 64, 7, 1),        # the only token outside the table
    (37, 1088, 500, 5),   # ragged piece count
    (64, 4096, 32000, 0),  # the decode batch's shape
    (64, 4096, 32000, 9),
    (300, 7168, 1000, 12),
    (5000, 1088, 300, 40),  # more rows than the grid has waves
    (33, 8192, 64, 3),    # the widest row
])
def test_embed_concat_bit_exact(M, d, vocab, n_bad):
    print(f"[case] embed_concat M={M} d={d} vocab={vocab} bad={n_bad}", flush=True)
    tokens, embed, fused = synth.make_embed_inputs(M, d, vocab, seed=M * 7 + d, n_bad=n_bad)
    got, bad = run(tokens, embed, fused)
    want, want_bad = oracle.embed_concat(tokens, embed, fused)
    assert got.shape == want.shape
    assert np.array_equal(got, want), f"{int(np.count_nonzero(got != want))} bf16 words differ"
    assert bad == want_bad == n_bad


def test_embed_concat_without_counter_and_repeatable():
    print("[case] embed_concat no counter", flush=True)
    tokens, embed, fused = synth.make_embed_inputs(100, 512, 50, seed=5, n_bad=4)
    a, _ = run(tokens, embed, fused, count=False)
    b, _ = run(tokens, embed, fused, count=False)
    assert np.array_equal(a, b) and np.array_equal(a, oracle.embed_concat(tokens, embed, fused)[0])


def test_embed_concat_prefill_shape_sampled():
    """The prefill batch's shape (M=32768, d=7168) in the launch the bench
    times: sampled rows, bit for bit."""
    print("[case] embed_concat M=32768 d=7168 (sampled rows)", flush=True)
    tokens, embed, fused = synth.make_embed_inputs(32768, 7168, 32000, seed=77, n_bad=16)
    got, bad = run(tokens, embed, fused)
    rows = np.unique(np.concatenate([np.arange(8), np.random.default_rng(1).choice(32768, 64, replace=False),
                                     np.arange(32760, 32768)]))
    want, want_bad = oracle.embed_concat(tokens[rows], embed, fused[rows])
    assert np.array_equal(got[rows], want)
    assert bad == 16
