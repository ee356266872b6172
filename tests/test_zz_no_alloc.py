"""eagle31_fuse_folded_noalloc (the folded step on the library's fixed
scratch array, for callers that cannot allocate) through the C ABI: the same
bits as eagle31_fuse_folded on the decode and the prefill path, two calls in a
row with the second smaller (the array keeps the first call's contents);
device free memory unchanged across its calls; a problem too large for the
array refused with EAGLE31_ERR_TOO_LARGE before anything is enqueued.
"""

import numpy as np
import pytest

import oracle
import synth
from parity import DevInputs, assert_parity, bf16_to_f64

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


def pair(dv, prepared, kind, eps, M):
    """The same call through eagle31_fuse_folded and the no-alloc entry point."""
    h = [x[:M] for x in dv.h]
    ref = e31().fuse_folded(h[0], h[1], h[2], kind, eps, *prepared)
    out = torch.empty_like(ref)
    e31().fuse_folded_noalloc(h[0], h[1], h[2], kind, eps, *prepared, out=out)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("cfg,d,Ms,kind,eps", [
    (2, 4096, (64, 16), LN, 1e-5),      # decode: the column-split kernel, 4 then 1 token tiles
    (2, 4096, (8, 6), LN, 1e-5),        # the column split, then packed token blocks (no scratch)
    (2, 4096, (4, 1), LN, 1e-5),        # packed token blocks, 4 then 1 token
    (3, 5120, (64, 17), RMS, 1e-6),
    (3, 5120, (128, 96), RMS, 1e-6),    # 65 to 128 tokens: the column-split kernel, 8 then 6 token tiles
    (None, 4096, (4096, 3072), LN, 1e-5),  # prefill without split-K (statistics in the array)
])
def test_noalloc_matches_fuse_folded(cfg, d, Ms, kind, eps):
    note(f"no-alloc cfg={cfg} d={d} Ms={Ms} kind={kind}")
    if cfg is None:
        w = synth.gen.custom_workload(d, (Ms[0],), seed_tag=4099)
        inp = synth.make_inputs(w, Ms[0])
    else:
        inp = synth.make_inputs(cfg, synth.CONFIGS[cfg].max_M)
    dv = DevInputs(inp)
    prepared = e31().fold_prepare(kind, dv.gamma, dv.beta, dv.W, dv.bias)
    outs = []
    for M in Ms:  # the second call is smaller than the first
        ref, out = pair(dv, prepared, kind, eps, M)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"no-alloc differs at M={M}"
        outs.append((M, out))
    # and both match the oracle (on a few rows for the prefill size)
    for M, out in outs:
        G = bf16_to_f64(out)
        rows = np.arange(M) if M <= 64 else np.unique(np.r_[0:8, M - 8:M, np.arange(8, M - 8, 97)])
        H = [oracle.decode_bf16(h[:M][rows]) for h in inp.h]
        g = [oracle.decode_bf16(x) for x in inp.gamma]
        b = None if (inp.beta is None or kind != LN) else [oracle.decode_bf16(x) for x in inp.beta]
        bias = None if inp.bias is None else oracle.decode_bf16(inp.bias)
        Y = oracle.fuse(H, kind, eps, g, b, oracle.decode_bf16(inp.W), bias)
        assert_parity(G[rows], Y, f"no-alloc d={d} M={M}")


def test_noalloc_refuses_decode_partials_over_the_array():
    """128 tokens at d=4096 (8 chunks x 8 token tiles of partials: 16 MiB plus
    counters and records) do not fit the 16 MiB array: refused before any
    launch, while 96 tokens (6 tiles) fit and match eagle31_fuse_folded."""
    note("no-alloc decode too large / fits")
    w = synth.gen.custom_workload(4096, (128,), seed_tag=4111)
    inp = synth.make_inputs(w, 128)
    dv = DevInputs(inp)
    prepared = e31().fold_prepare(LN, dv.gamma, dv.beta, dv.W, dv.bias)
    out = torch.empty((128, 4096), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(e31().Eagle31Error) as ei:
        e31().fuse_folded_noalloc(dv.h[0], dv.h[1], dv.h[2], LN, 1e-5, *prepared, out=out)
    assert ei.value.status == e31()._capi.ERR_TOO_LARGE
    ref, got = pair(dv, prepared, LN, 1e-5, 96)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_noalloc_allocates_nothing():
    """After a first call (which looks up the array and zeroes its counters),
    further calls leave the device's free memory unchanged."""
    note("no-alloc free memory")
    inp = synth.make_inputs(2, 64)
    dv = DevInputs(inp)
    prepared = e31().fold_prepare(LN, dv.gamma, dv.beta, dv.W, dv.bias)
    outs = [torch.empty((M, inp.d), dtype=torch.bfloat16, device="cuda") for M in (64, 8, 1)]
    e31().fuse_folded_noalloc(dv.h[0], dv.h[1], dv.h[2], LN, 1e-5, *prepared, out=outs[0])
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        for o in outs:
            M = o.shape[0]
            e31().fuse_folded_noalloc(dv.h[0][:M], dv.h[1][:M], dv.h[2][:M], LN, 1e-5, *prepared, out=o)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, f"device free memory changed by {free0 - free1} bytes"


def test_noalloc_refuses_too_large():
    """d=8192, M=512 splits K over 3 chunks: 48 MiB of partials, more than the
    array holds; refused before any launch, and the next call is unaffected."""
    note("no-alloc too large")
    assert e31().noalloc_scratch_bytes() == 16 << 20
    d, M = 8192, 512
    h = [torch.zeros((M, d), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    wf = torch.zeros(e31().ops.folded_shape(d), dtype=torch.bfloat16, device="cuda")
    u = torch.zeros((3, d), dtype=torch.float32, device="cuda")
    c = torch.zeros((d,), dtype=torch.float32, device="cuda")
    out = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(e31().Eagle31Error) as ei:
        e31().fuse_folded_noalloc(h[0], h[1], h[2], LN, 1e-5, wf, u, c, out=out)
    assert ei.value.status == e31()._capi.ERR_TOO_LARGE
    # a call that fits still works right after
    inp = synth.make_inputs(1, 64)
    dv = DevInputs(inp)
    prepared = e31().fold_prepare(LN, dv.gamma, dv.beta, dv.W, dv.bias)
    ref, got = pair(dv, prepared, LN, 1e-5, 64)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
