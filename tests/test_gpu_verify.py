"""eagle31_verify_accept against the oracle (oracle/verify64.py) through the
C ABI: the number of drafts kept and the emitted token must be identical
(integers decided by the definition in exact arithmetic, the keep test in
float32 on both sides).  Seeded batches at several vocabulary sizes (one and
several chunks per row, ragged tails, sizes that are not multiples of four),
q = p (every draft kept, bonus draws), all-rejected rows, residuals that are
all zero, zero-probability drafts, ids outside the vocabulary, invalid rows
(NaN, values above 1, u_res outside [0, 1)), tiny and subnormal weights,
u_res on exact prefix boundaries; repeatability.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def run(p, q, draft, u_acc, u_res):
    n, t = e31().verify_accept(dev(p), dev(q), dev(draft.astype(np.int32)), dev(u_acc), dev(u_res))
    torch.cuda.synchronize()
    return n.cpu().numpy(), t.cpu().numpy()


def check(p, q, draft, u_acc, u_res, what):
    n, t = run(p, q, draft, u_acc, u_res)
    n_o, t_o = oracle.verify_accept(p, q, draft, u_acc, u_res)
    bad_n = np.nonzero(n != n_o)[0]
    bad_t = np.nonzero(t != t_o)[0]
    print(f"[verify] {what}: B={len(n)} kept {n.tolist()[:8]}... emitted {t.tolist()[:6]}...; "
          f"mismatches n {len(bad_n)} t {len(bad_t)}", flush=True)
    assert len(bad_n) == 0, f"{what}: n_accepted differs at {bad_n[:8]} ({n[bad_n[:8]]} vs {n_o[bad_n[:8]]})"
    assert len(bad_t) == 0, f"{what}: next_token differs at {bad_t[:8]} ({t[bad_t[:8]]} vs {t_o[bad_t[:8]]})"
    return n, t


@pytest.mark.parametrize("B,N,V,spread", [(64, 4, 32000, 0.5), (16, 8, 32000, 1.0), (8, 4, 128256, 0.5),
                                          (5, 3, 4099, 1.0), (3, 2, 1027, 0.3), (33, 1, 8191, 1.0),
                                          (1, 64, 4096, 0.5), (7, 5, 5, 1.0), (16, 3, 6143, 1.0)])
def test_verify_random_batches(B, N, V, spread):
    note(f"verify random B={B} N={N} V={V}")
    p, q, draft, u_acc, u_res = synth.make_verify_inputs(B, N, V, seed=B * 1000 + V, spread=spread)
    n, _ = check(p, q, draft, u_acc, u_res, f"random B={B} N={N} V={V}")
    # repeatable
    n2, t2 = run(p, q, draft, u_acc, u_res)
    assert np.array_equal(n, n2)


@pytest.mark.parametrize("B,N,V,L", [(8, 4, 128256, 4096), (64, 4, 151936, 8192), (2, 2, 2_100_000, 16384)])
def test_verify_each_chunk_size(B, N, V, L):
    """Rows split into 4096-, 8192- and 16384-token chunks (the last searches
    its quarter with the general loop); rows are independent, so a sample of
    them is checked against the oracle on the same inputs."""
    note(f"verify chunk size B={B} N={N} V={V}")
    assert e31().verify_chunking(B, N, V) == (-(-V // L), L)
    p, q, draft, u_acc, u_res = synth.make_verify_inputs(B, N, V, seed=V + B, spread=0.5)
    n, t = run(p, q, draft, u_acc, u_res)
    rows = np.unique(np.concatenate([[0, B - 1], np.random.default_rng(V).choice(B, min(B, 14), replace=False)]))
    n_o, t_o = oracle.verify_accept(p[rows], q[rows], draft[rows], u_acc[rows], u_res[rows])
    print(f"[verify] chunk size {L}: rows {rows.tolist()} kept {n[rows].tolist()} emitted {t[rows].tolist()}", flush=True)
    assert np.array_equal(n[rows], n_o), (n[rows], n_o)
    assert np.array_equal(t[rows], t_o), (t[rows], t_o)
    assert (t[rows] >= 0).all()


def test_verify_q_equals_p_keeps_every_draft():
    note("verify q = p")
    B, N, V = 16, 4, 32000
    p, q, draft, u_acc, u_res = synth.make_verify_inputs(B, N, V, seed=5)
    q[:, :N] = p
    n, _ = check(p, q, draft, u_acc, u_res, "q = p")
    assert np.all(n == N)


def test_verify_all_rejected_and_zero_residual():
    """Row 0: the first draft has q = 0 < p, so it is rejected (j = 0) and the
    residual is drawn.  Row 1: q = p and the draft has p = q = 0, rejected at
    0 with an all-zero residual, so the token comes from q_0 itself.  Row 2:
    an id outside the vocabulary at position 1.  Row 3: p(d) = 0 < q(d), kept."""
    note("verify all-rejected / zero residual / bad ids")
    B, N, V = 4, 3, 2048
    p, q, draft, u_acc, u_res = synth.make_verify_inputs(B, N, V, seed=9, spread=0.2)
    q[0, 0, draft[0, 0]] = 0.0
    q[1, :N] = p[1]
    p[1, 0, 7] = 0.0
    q[1, 0, 7] = 0.0
    draft[1, 0] = 7
    draft[2, 1] = V + 5
    p[3, 0, 11] = 0.0
    draft[3, 0] = 11
    n, t = check(p, q, draft, u_acc, u_res, "special rows")
    assert n[0] == 0 and n[1] == 0 and n[2] <= 1


def test_verify_invalid_rows_give_no_token():
    note("verify invalid rows")
    B, N, V = 6, 2, 3000
    p, q, draft, u_acc, u_res = synth.make_verify_inputs(B, N, V, seed=11, spread=0.1)
    u_acc[:] = 0.0             # every draft with p > 0 kept unless q(d) = 0
    u_acc[0, 0] = 2.0          # row 0: 2 p(d) < q(d) fails for most d -> a residual row
    q[0, 0, 100] = np.nan      # ... which holds a NaN
    q[1, N, 200] = 1.5         # row 1: the bonus row holds a value above 1
    q[2, N, :] = 0.0           # row 2: the bonus row is all zero
    u_res[3] = 1.0             # row 3: u_res outside [0, 1)
    u_res[4] = -0.5
    n, t = check(p, q, draft, u_acc, u_res, "invalid rows")
    assert t[1] == -1 and t[2] == -1 and t[3] == -1 and t[4] == -1


def test_verify_tiny_subnormal_weights_and_boundaries():
    """Bonus rows built from tiny (2^-100), subnormal and ordinary weights, and
    u_res chosen so that u_res * total falls exactly on a prefix sum (the
    strict inequality decides); float64 running sums would get some wrong."""
    note("verify tiny / subnormal / boundaries")
    B, N, V = 12, 1, 1030
    rng = np.random.default_rng(13)
    p = np.zeros((B, N, V), dtype=np.float32)
    q = np.zeros((B, N + 1, V), dtype=np.float32)
    draft = np.zeros((B, N), dtype=np.int32)
    p[:, 0, 0] = 1.0
    q[:, 0, 0] = 1.0           # the draft (token 0) is always kept: the bonus row is drawn
    u_acc = np.zeros((B, N), dtype=np.float32)
    u_res = rng.random(B, dtype=np.float32)
    for b in range(B):
        w = rng.random(V).astype(np.float32) * np.float32(1e-3)
        kind = rng.integers(0, 4, size=V)
        w[kind == 1] = np.float32(2.0 ** -100)
        w[kind == 2] = np.float32(1e-42)
        w[kind == 3] = 0.0
        q[b, N] = w
    # exact boundaries: w = (.5, 2^-100, .5) with u = .5 -> token 1 (the tiny one)
    q[0, N, :] = 0.0
    q[0, N, 10], q[0, N, 500], q[0, N, 1020] = 0.5, 2.0 ** -100, 0.5
    u_res[0] = 0.5
    # u_res * total equal to a prefix: w = 0.25 everywhere on 4 tokens, u = .5
    q[1, N, :] = 0.0
    q[1, N, [3, 300, 600, 900]] = 0.25
    u_res[1] = 0.5
    # u_res = 0: the first token with a positive weight
    u_res[2] = 0.0
    _, t = check(p, q, draft, u_acc, u_res, "tiny / subnormal / boundary")
    assert t[0] == 500 and t[1] == 600
