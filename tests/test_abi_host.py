"""The C ABI on the host (no GPU needed): the library loads, exports every
symbol the header declares, and rejects bad arguments before any HIP call.

Only argument validation and M == 0 are exercised here: every call below
returns before the library touches the HIP runtime.
"""

import ctypes
import os
import re

import pytest

import eagle_draft_feature_amd as e31
from eagle_draft_feature_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eagle31.h")

# fake, 16-byte aligned device addresses: validation never dereferences them
H0, H1, H2, WP, BP, OUT = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(eagle31_[a-z_]+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_symbol():
    L = e31.lib()
    syms = declared_symbols()
    assert len(syms) >= 11
    for s in syms:
        assert hasattr(L, s), f"{s} declared in eagle31.h but not exported"
    assert set(syms) == set(_capi.SIGNATURES), "binding signatures out of sync with the header"


def _fuse(**kw):
    a = dict(h0=H0, h1=H1, h2=H2, M=4, d=128, norm=1, eps=1e-5, g=None, b=None, W=WP, bias=BP, out=OUT)
    a.update(kw)
    return e31.lib().eagle31_fuse(a["h0"], a["h1"], a["h2"], a["M"], a["d"], a["norm"], a["eps"], a["g"], a["b"],
                                  a["W"], a["bias"], a["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=100), _capi.ERR_SHAPE),
    (dict(d=0), _capi.ERR_SHAPE),
    (dict(d=-64), _capi.ERR_SHAPE),
    (dict(d=65536 + 64), _capi.ERR_SHAPE),
    (dict(M=-1), _capi.ERR_SHAPE),
    (dict(M=16777217), _capi.ERR_SHAPE),
    (dict(norm=3), _capi.ERR_NORM_KIND),
    (dict(norm=-1), _capi.ERR_NORM_KIND),
    (dict(eps=-1e-5), _capi.ERR_EPS),
    (dict(eps=float("nan")), _capi.ERR_EPS),
    (dict(eps=float("inf")), _capi.ERR_EPS),
    (dict(h0=None), _capi.ERR_NULL),
    (dict(h2=None), _capi.ERR_NULL),
    (dict(out=None), _capi.ERR_NULL),
    (dict(W=None), _capi.ERR_NULL),
    (dict(h1=H1 + 2), _capi.ERR_ALIGN),
    (dict(out=OUT + 8), _capi.ERR_ALIGN),
    (dict(W=WP + 4), _capi.ERR_ALIGN),
    (dict(bias=BP + 2), _capi.ERR_ALIGN),
    (dict(out=H1 + 256), _capi.ERR_ALIAS),
    (dict(out=WP + 1024), _capi.ERR_ALIAS),
])
def test_fuse_rejects_bad_arguments(kw, code):
    assert _fuse(**kw) == code


def test_fuse_M0_is_a_no_op():
    assert _fuse(M=0, h0=None, h1=None, h2=None, out=None) == _capi.OK


def test_fuse_gamma_beta_alignment_checked():
    g, keep = _capi.ptr_array3([0x700000, 0x700102, 0x700200])
    assert _fuse(g=g) == _capi.ERR_ALIGN
    b, keep2 = _capi.ptr_array3([0x800000, None, 0x800208])
    assert _fuse(b=b) == _capi.ERR_ALIGN
    # beta is ignored for RMSNorm, gamma for NONE
    assert _fuse(b=b, norm=2, M=0, h0=None, h1=None, h2=None, out=None) == _capi.OK
    assert _fuse(g=g, norm=0, M=0, h0=None, h1=None, h2=None, out=None) == _capi.OK


def test_folded_and_prepare_validation():
    L = e31.lib()
    f = L.eagle31_fuse_folded
    assert f(H0, H1, H2, 4, 100, 1, 1e-5, WP, BP, 0x900000, OUT, None) == _capi.ERR_SHAPE
    assert f(H0, H1, H2, 4, 128, 1, 1e-5, None, BP, 0x900000, OUT, None) == _capi.ERR_NULL
    assert f(H0, H1, H2, 4, 128, 1, 1e-5, WP, BP + 4, 0x900000, OUT, None) == _capi.ERR_ALIGN
    assert f(H0, H1, H2, 4, 128, 1, 1e-5, WP, BP, 0x900000, WP + 16, None) == _capi.ERR_ALIAS
    assert f(None, None, None, 0, 128, 1, 1e-5, WP, BP, 0x900000, None, None) == _capi.OK
    p = L.eagle31_fold_prepare
    assert p(100, 1, None, None, WP, None, OUT, BP, 0x900000, None) == _capi.ERR_SHAPE
    assert p(128, 1, None, None, None, None, OUT, BP, 0x900000, None) == _capi.ERR_NULL
    assert p(128, 1, None, None, WP, None, WP + 64, BP, 0x900000, None) == _capi.ERR_ALIAS
    assert p(128, 7, None, None, WP, None, OUT, BP, 0x900000, None) == _capi.ERR_NORM_KIND


def test_workspace_entry_points_validation():
    L = e31.lib()
    assert L.eagle31_workspace_size(64, 4096, 1) > 0
    assert L.eagle31_workspace_size(32768, 7168, 1) >= 3 * 7168 * 7168 * 2  # folded weight of the large-M path
    assert L.eagle31_workspace_size(64, 100, 1) == 0
    assert L.eagle31_workspace_init(None, 1024, None) == _capi.ERR_NULL
    assert L.eagle31_workspace_init(0x100010, 1024, None) == _capi.ERR_ALIGN
    fw = L.eagle31_fuse_ws
    assert fw(H0, H1, H2, 4, 128, 1, 1e-5, None, None, WP, BP, OUT, None, 0, None) == _capi.ERR_WORKSPACE
    assert fw(H0, H1, H2, 4, 128, 1, 1e-5, None, None, WP, BP, OUT, 0xA00000, 16, None) == _capi.ERR_WORKSPACE
    assert fw(H0, H1, H2, 4, 128, 1, 1e-5, None, None, WP, BP, OUT, 0xA00010, 1 << 30, None) == _capi.ERR_ALIGN
    assert fw(H0, H1, H2, 4, 100, 1, 1e-5, None, None, WP, BP, OUT, 0xA00000, 1 << 30, None) == _capi.ERR_SHAPE


def test_row_stats_validation():
    L = e31.lib()
    r = L.eagle31_row_stats
    assert r(H0, H1, H2, 4, 96, 1, 1e-5, OUT, BP, None) == _capi.ERR_SHAPE
    assert r(H0, None, H2, 4, 128, 1, 1e-5, OUT, BP, None) == _capi.ERR_NULL
    assert r(H0, H1, H2, 4, 128, 1, 1e-5, OUT + 4, BP, None) == _capi.ERR_ALIGN
    assert r(None, None, None, 0, 128, 1, 1e-5, None, None, None) == _capi.OK


def test_status_strings_and_last_hip_error():
    L = e31.lib()
    for code in _capi.STATUS_NAMES:
        s = L.eagle31_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert L.eagle31_status_string(-99) == b"unknown status"
    assert L.eagle31_last_hip_error() == 0


def test_python_wrapper_checks_types_without_gpu():
    import torch
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        e31.fuse(x, x, x, "ln", 1e-5, None, None, torch.zeros(384, 128, dtype=torch.bfloat16), None)
    with pytest.raises(TypeError):
        e31.fuse(x.float(), x, x, "ln", 1e-5, None, None, x, None)


def test_stats_recompute_hook_is_host_only():
    """The test hook only sets a process-wide flag read at the next launch:
    it returns OK without touching the GPU, and can be switched back."""
    L = e31.lib()
    assert L.eagle31_debug_stats_recompute(1) == 0
    assert L.eagle31_debug_stats_recompute(0) == 0
    e31.debug_stats_recompute(True)
    e31.debug_stats_recompute(False)


def _norm_out(x=H0, M=64, d=4096, norm=1, eps=1e-5, g=WP, b=BP, out=OUT):
    return e31.lib().eagle31_norm_output(x, M, d, norm, eps, g, b, out, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=8192 + 64), _capi.ERR_SHAPE),  # the post-norm kernel's row limit
    (dict(d=96), _capi.ERR_SHAPE),
    (dict(M=-1), _capi.ERR_SHAPE),
    (dict(norm=7), _capi.ERR_NORM_KIND),
    (dict(eps=float("nan")), _capi.ERR_EPS),
    (dict(x=None), _capi.ERR_NULL),
    (dict(out=None), _capi.ERR_NULL),
    (dict(x=H0 + 2), _capi.ERR_ALIGN),
    (dict(out=OUT + 8), _capi.ERR_ALIGN),
    (dict(g=WP + 4), _capi.ERR_ALIGN),
    (dict(b=BP + 2), _capi.ERR_ALIGN),
    (dict(out=H0 + 16), _capi.ERR_ALIAS),  # partial overlap with x
    (dict(out=WP - 64 * 4096 * 2 + 16), _capi.ERR_ALIAS),  # out's last row runs into gamma
    (dict(out=BP - 1024), _capi.ERR_ALIAS),
])
def test_norm_output_rejects_bad_arguments(kw, code):
    assert _norm_out(**kw) == code


def test_norm_output_host_rules_for_parameters():
    """M == 0 launches nothing; beta's alignment and overlap are not checked
    where beta is unused (RMSNorm), nor gamma's for NONE."""
    assert _norm_out(M=0) == _capi.OK
    assert _norm_out(M=0, x=None, out=None) == _capi.OK
    assert _norm_out(M=0, norm=2, b=BP + 2, d=8192 + 64) == _capi.ERR_SHAPE


def _ecat(tok=0x700000, M=64, d=4096, vocab=16, e=WP, f=H1, dst=OUT, bad=None):
    # regions: embed [WP, WP + 128 KiB), fused [H1, H1 + 512 KiB), dst [OUT, OUT + 1 MiB), tokens at 0x700000
    return e31.lib().eagle31_embed_concat(tok, M, d, vocab, e, f, dst, bad, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=8192 + 64), _capi.ERR_SHAPE),
    (dict(d=96), _capi.ERR_SHAPE),
    (dict(vocab=0), _capi.ERR_SHAPE),
    (dict(vocab=2 ** 31), _capi.ERR_SHAPE),
    (dict(M=-1), _capi.ERR_SHAPE),
    (dict(tok=None), _capi.ERR_NULL),
    (dict(e=None), _capi.ERR_NULL),
    (dict(f=None, e=None), _capi.ERR_NULL),   # fused may be NULL (embedding half only), embed may not
    (dict(f=None, e=WP + 8), _capi.ERR_ALIGN),
    (dict(f=H1 + 4), _capi.ERR_ALIGN),
    (dict(dst=None), _capi.ERR_NULL),
    (dict(tok=0x700002), _capi.ERR_ALIGN),
    (dict(bad=0x700001), _capi.ERR_ALIGN),
    (dict(e=WP + 8), _capi.ERR_ALIGN),
    (dict(dst=OUT + 4), _capi.ERR_ALIGN),
    (dict(dst=H1 - 1024), _capi.ERR_ALIAS),  # dst runs into the fused feature
    (dict(tok=OUT + 64), _capi.ERR_ALIAS),
    (dict(bad=OUT + 1024), _capi.ERR_ALIAS),
    (dict(M=0, tok=None, dst=None), _capi.OK),
    (dict(e=OUT + 4096 * 2 * 4), _capi.ERR_ALIAS),  # the table starts inside dst
])
def test_embed_concat_rejects_bad_arguments(kw, code):
    assert _ecat(**kw) == code


# verify / accept: fake device addresses, 16-byte aligned; B=4, N=2, V=1000
VP, VQ, VD, VUA, VUR, VN, VT = 0x1000000, 0x2000000, 0x3000000, 0x3100000, 0x3200000, 0x3300000, 0x3400000


def _verify(**kw):
    a = dict(p=VP, q=VQ, d=VD, ua=VUA, ur=VUR, B=4, N=2, V=1000, n=VN, t=VT)
    a.update(kw)
    return e31.lib().eagle31_verify_accept(a["p"], a["q"], a["d"], a["ua"], a["ur"], a["B"], a["N"], a["V"], a["n"],
                                           a["t"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), _capi.ERR_SHAPE),
    (dict(B=4097), _capi.ERR_SHAPE),
    (dict(N=0), _capi.ERR_SHAPE),
    (dict(N=65), _capi.ERR_SHAPE),
    (dict(V=0), _capi.ERR_SHAPE),
    (dict(V=(1 << 26) + 1), _capi.ERR_SHAPE),
    (dict(p=None), _capi.ERR_NULL),
    (dict(ur=None), _capi.ERR_NULL),
    (dict(t=None), _capi.ERR_NULL),
    (dict(q=VQ + 2), _capi.ERR_ALIGN),
    (dict(d=VD + 1), _capi.ERR_ALIGN),
    (dict(n=VN + 2), _capi.ERR_ALIGN),
    (dict(n=VP + 4 * 1000), _capi.ERR_ALIAS),     # inside p
    (dict(t=VQ + 8), _capi.ERR_ALIAS),            # inside q
    (dict(t=VN + 8), _capi.ERR_ALIAS),            # overlaps n_accepted
    (dict(n=VUA + 4), _capi.ERR_ALIAS),           # inside u_acc
    (dict(B=0, p=None, t=None), _capi.OK),        # nothing to do
])
def test_verify_accept_rejects_bad_arguments(kw, code):
    assert _verify(**kw) == code


def _chunking(B, N, V):
    c, t = ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = e31.lib().eagle31_verify_chunking(B, N, V, ctypes.byref(c), ctypes.byref(t))
    return st, c.value, t.value


@pytest.mark.parametrize("B,N,V,want", [
    (64, 4, 32000, (4, 8192)),
    (64, 4, 128256, (16, 8192)),
    (64, 4, 151936, (19, 8192)),
    (16, 4, 32000, (16, 2048)),
    (8, 4, 128256, (32, 4096)),
    (1, 1, 2_100_000, (129, 16384)),
    (1, 1, 5, (1, 2048)),
    (4096, 1, 8192, (1, 8192)),
])
def test_verify_chunking_examples(B, N, V, want):
    st, c, t = _chunking(B, N, V)
    assert st == _capi.OK and (c, t) == want
    assert e31.verify_chunking(B, N, V) == want


def test_verify_chunking_rules():
    """The chunk plan for a grid of shapes: pieces of 2048 * 2^k tokens that
    cover the row, at most 256 per row; 8192 tokens at most unless the row
    needs more than 256 pieces; the smallest piece that keeps B * chunks at or
    below 256 (one workgroup per CU)."""
    def C(V, L):
        return -(-V // L)
    for B in (1, 3, 64, 255, 1000, 4096):
        for V in (1, 5, 2047, 2048, 2049, 32000, 128256, 151936, 262144, 524289, 2_100_000, 1 << 26):
            st, c, L = _chunking(B, 4, V)
            assert st == _capi.OK
            assert L >= 2048 and L % 2048 == 0 and (L & (L - 1)) == 0
            assert c == C(V, L) and (c - 1) * L < V <= c * L and c <= 256
            if L > 8192:
                assert C(V, L // 2) > 256
            elif L > 2048:
                assert C(V, L // 2) > 256 or B * C(V, L // 2) > 256
    assert _chunking(0, 1, 10)[0] == _capi.ERR_SHAPE
    assert _chunking(1, 0, 10)[0] == _capi.ERR_SHAPE
    assert _chunking(1, 1, (1 << 26) + 1)[0] == _capi.ERR_SHAPE
    assert e31.lib().eagle31_verify_chunking(1, 1, 10, None, ctypes.byref(ctypes.c_int32())) == _capi.ERR_NULL


# strided / indexed rows: fake device addresses; d=128, states 16 MiB apart, out and index elsewhere
RH0, RH1, RH2, ROUT, RIDX, RWF, RU, RC = 0x10000000, 0x11000000, 0x12000000, 0x13000000, 0x14000000, 0x15000000, \
    0x16000000, 0x17000000


def _frows(**kw):
    a = dict(h0=RH0, h1=RH1, h2=RH2, ld=(128, 128, 128), idx=None, n_src=64, M=16, d=128, norm=1, eps=1e-5,
             out=ROUT, ld_out=128, wf=RWF, u=RU, c=RC)
    a.update(kw)
    ld = None if a["ld"] is None else (ctypes.c_int64 * 3)(*a["ld"])
    return e31.lib().eagle31_fuse_folded_rows(a["h0"], a["h1"], a["h2"], ld, a["idx"], a["n_src"], a["M"], a["d"],
                                              a["norm"], a["eps"], a["wf"], a["u"], a["c"], a["out"], a["ld_out"],
                                              None)


def _srows(**kw):
    a = dict(h0=RH0, h1=RH1, h2=RH2, ld=(128, 128, 128), idx=None, n_src=64, M=16, d=128, W=RWF, out=ROUT,
             ld_out=128)
    a.update(kw)
    ld = None if a["ld"] is None else (ctypes.c_int64 * 3)(*a["ld"])
    return e31.lib().eagle31_fuse_rows(a["h0"], a["h1"], a["h2"], ld, a["idx"], a["n_src"], a["M"], a["d"], 1, 1e-5,
                                       None, None, a["W"], None, a["out"], a["ld_out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ld=(120, 128, 128)), _capi.ERR_SHAPE),          # below d
    (dict(ld=(128, 132, 128)), _capi.ERR_SHAPE),          # not a multiple of 8
    (dict(ld=(128, 128, (1 << 22) + 8)), _capi.ERR_SHAPE),
    (dict(ld_out=64), _capi.ERR_SHAPE),
    (dict(ld_out=136 + 4), _capi.ERR_SHAPE),
    (dict(n_src=0), _capi.ERR_SHAPE),
    (dict(n_src=15), _capi.ERR_SHAPE),                    # fewer rows than tokens, no index list
    (dict(n_src=2 ** 31), _capi.ERR_SHAPE),
    (dict(idx=RIDX, n_src=(1 << 22) // 2 + 1, ld=(1 << 11, 128, 128)), _capi.ERR_SHAPE),  # > 4 GiB reachable
    (dict(M=-1), _capi.ERR_SHAPE),
    (dict(d=100), _capi.ERR_SHAPE),
    (dict(norm=5), _capi.ERR_NORM_KIND),
    (dict(h1=None), _capi.ERR_NULL),
    (dict(out=None), _capi.ERR_NULL),
    (dict(wf=None), _capi.ERR_NULL),
    (dict(h2=RH2 + 8), _capi.ERR_ALIGN),
    (dict(out=ROUT + 2), _capi.ERR_ALIGN),
    (dict(idx=RIDX + 2), _capi.ERR_ALIGN),
    (dict(out=RH0 + 63 * 256 * 2), _capi.ERR_ALIAS),   # inside h_low's last row at ld = 256
    (dict(out=RIDX - 16 * 128 * 2 + 64, idx=RIDX), _capi.ERR_ALIAS),  # runs into the index list
    (dict(out=RWF - 1024), _capi.ERR_ALIAS),           # runs into the folded weight
    (dict(M=0, h0=None, out=None), _capi.OK),
])
def test_fuse_folded_rows_rejects_bad_arguments(kw, code):
    if kw.get("out") == RH0 + 63 * 256 * 2:
        kw = dict(kw, ld=(256, 128, 128))
    assert _frows(**kw) == code


def test_fuse_rows_strided_extent_checks():
    # out 1 KiB past h_low's start: overlaps once h_low rows are 1024 elements apart
    assert _srows(out=RH0 + 64 * 128 * 2 + 1024, ld=(1024, 128, 128)) == _capi.ERR_ALIAS
    assert _srows(ld=(128, 128, 100)) == _capi.ERR_SHAPE
    assert _srows(W=None) == _capi.ERR_NULL
    assert _srows(idx=RIDX + 1) == _capi.ERR_ALIGN
    # out rows 2d apart reach ((M - 1) * 2d + d) elements: into h0 when h0 starts there
    assert _srows(out=RH0 - 15 * 256 * 2, ld_out=256) == _capi.ERR_ALIAS
