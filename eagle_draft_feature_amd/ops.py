"""torch-facing wrappers of the C ABI: argument checks and pointer marshalling.

torch provides device memory and the current HIP stream; nothing here
computes.  All tensors must be contiguous bfloat16 (statistics and folded
vectors float32) on the same GPU, except the hidden states and output of
fuse_rows / fuse_folded_rows: 2-D views whose rows may be any number of
elements apart (unit column stride).
"""

from __future__ import annotations

from typing import Optional, Sequence, Union

import torch

from . import _capi
from ._capi import check, lib, ptr_array3

_NAMES = {"none": _capi.NORM_NONE, "layernorm": _capi.NORM_LAYERNORM, "ln": _capi.NORM_LAYERNORM,
          "rmsnorm": _capi.NORM_RMSNORM, "rms": _capi.NORM_RMSNORM}


def norm_kind(kind: Union[int, str]) -> int:
    if isinstance(kind, str):
        return _NAMES[kind.lower()]
    return int(kind)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _want(t: torch.Tensor, name: str, dtype=torch.bfloat16, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _vec3(ts: Optional[Sequence[Optional[torch.Tensor]]], name: str, d: int, device):
    if ts is None:
        return None
    if len(ts) != 3:
        raise ValueError(f"{name} needs three entries (low, mid, high)")
    for i, t in enumerate(ts):
        if t is not None:
            _want(t, f"{name}[{i}]", shape=(d,), device=device)
    return ptr_array3([_ptr(t) for t in ts])


def _states(h_low, h_mid, h_high):
    _want(h_low, "h_low")
    if h_low.dim() != 2:
        raise ValueError("hidden states must be [M, d]")
    M, d = h_low.shape
    for nm, t in (("h_mid", h_mid), ("h_high", h_high)):
        _want(t, nm, shape=(M, d), device=h_low.device)
    return M, d, h_low.device


def fuse(h_low: torch.Tensor, h_mid: torch.Tensor, h_high: torch.Tensor, norm: Union[int, str], eps: float,
         gammas: Optional[Sequence[Optional[torch.Tensor]]], betas: Optional[Sequence[Optional[torch.Tensor]]],
         W: torch.Tensor, bias: Optional[torch.Tensor], out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[M, d] = [norm(h_low) | norm(h_mid) | norm(h_high)] @ W + bias (eagle31_fuse)."""
    M, d, dev = _states(h_low, h_mid, h_high)
    _want(W, "W", shape=(3 * d, d), device=dev)
    if bias is not None:
        _want(bias, "bias", shape=(d,), device=dev)
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    _want(out, "out", shape=(M, d), device=dev)
    g = _vec3(gammas, "gammas", d, dev)
    b = _vec3(betas, "betas", d, dev)
    st = lib().eagle31_fuse(_ptr(h_low), _ptr(h_mid), _ptr(h_high), M, d, norm_kind(norm), float(eps),
                            g[0] if g else None, b[0] if b else None, _ptr(W), _ptr(bias), _ptr(out),
                            _stream(h_low))
    check("eagle31_fuse", st)
    return out


def workspace_size(M: int, d: int, norm: Union[int, str]) -> int:
    return int(lib().eagle31_workspace_size(M, d, norm_kind(norm)))


def workspace_init(ws: torch.Tensor) -> None:
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    check("eagle31_workspace_init", lib().eagle31_workspace_init(_ptr(ws), ws.numel() * ws.element_size(),
                                                                  _stream(ws)))


def fuse_ws(h_low, h_mid, h_high, norm, eps, gammas, betas, W, bias, workspace: torch.Tensor,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """eagle31_fuse_ws: as fuse(), with a caller workspace (see workspace_size / workspace_init)."""
    M, d, dev = _states(h_low, h_mid, h_high)
    _want(W, "W", shape=(3 * d, d), device=dev)
    if bias is not None:
        _want(bias, "bias", shape=(d,), device=dev)
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    _want(out, "out", shape=(M, d), device=dev)
    g = _vec3(gammas, "gammas", d, dev)
    b = _vec3(betas, "betas", d, dev)
    st = lib().eagle31_fuse_ws(_ptr(h_low), _ptr(h_mid), _ptr(h_high), M, d, norm_kind(norm), float(eps),
                               g[0] if g else None, b[0] if b else None, _ptr(W), _ptr(bias), _ptr(out),
                               _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(h_low))
    check("eagle31_fuse_ws", st)
    return out


def folded_shape(d: int):
    """Shape given to the folded weight: [d/16, 3d/32, 64, 8] bf16, i.e. column
    block, k-step of 32, MFMA lane, 8 consecutive k (1 KiB per tile)."""
    return (d // 16, 3 * d // 32, 64, 8)


def fold_prepare(norm: Union[int, str], gammas, betas, W: torch.Tensor, bias: Optional[torch.Tensor]):
    """eagle31_fold_prepare: returns (w_folded bf16 tiles, u [3, d] f32, c [d] f32)."""
    _want(W, "W")
    if W.dim() != 2 or W.shape[0] != 3 * W.shape[1]:
        raise ValueError("W must be [3d, d]")
    d = W.shape[1]
    dev = W.device
    if bias is not None:
        _want(bias, "bias", shape=(d,), device=dev)
    wf = torch.empty(folded_shape(d), dtype=torch.bfloat16, device=dev)
    u = torch.empty((3, d), dtype=torch.float32, device=dev)
    c = torch.empty((d,), dtype=torch.float32, device=dev)
    g = _vec3(gammas, "gammas", d, dev)
    b = _vec3(betas, "betas", d, dev)
    st = lib().eagle31_fold_prepare(d, norm_kind(norm), g[0] if g else None, b[0] if b else None, _ptr(W),
                                    _ptr(bias), _ptr(wf), _ptr(u), _ptr(c), _stream(W))
    check("eagle31_fold_prepare", st)
    return wf, u, c


def fuse_folded(h_low, h_mid, h_high, norm, eps, w_folded: torch.Tensor, u: torch.Tensor, c: torch.Tensor,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """eagle31_fuse_folded (or _ws when a workspace is given) on prepared weights."""
    M, d, dev = _states(h_low, h_mid, h_high)
    _want(w_folded, "w_folded", shape=folded_shape(d), device=dev)
    _want(u, "u", dtype=torch.float32, shape=(3, d), device=dev)
    _want(c, "c", dtype=torch.float32, shape=(d,), device=dev)
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    _want(out, "out", shape=(M, d), device=dev)
    if workspace is None:
        st = lib().eagle31_fuse_folded(_ptr(h_low), _ptr(h_mid), _ptr(h_high), M, d, norm_kind(norm), float(eps),
                                       _ptr(w_folded), _ptr(u), _ptr(c), _ptr(out), _stream(h_low))
        check("eagle31_fuse_folded", st)
    else:
        st = lib().eagle31_fuse_folded_ws(_ptr(h_low), _ptr(h_mid), _ptr(h_high), M, d, norm_kind(norm),
                                          float(eps), _ptr(w_folded), _ptr(u), _ptr(c), _ptr(out), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(h_low))
        check("eagle31_fuse_folded_ws", st)
    return out


def _rows_view(t: torch.Tensor, name: str, d: Optional[int] = None, device=None):
    """A [rows, d] bf16 view with unit column stride; returns its row stride."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be torch.bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D view with unit column stride")
    if d is not None and t.shape[1] != d:
        raise ValueError(f"{name} has {t.shape[1]} columns, expected {d}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def _row_args(h_low, h_mid, h_high, row_index, out):
    import ctypes
    d = h_low.shape[1] if h_low.dim() == 2 else -1
    ld = [_rows_view(t, nm, d, h_low.device) for nm, t in (("h_low", h_low), ("h_mid", h_mid), ("h_high", h_high))]
    n_src = h_low.shape[0]
    if h_mid.shape[0] != n_src or h_high.shape[0] != n_src:
        raise ValueError("the three states must hold the same number of rows")
    dev = h_low.device
    if row_index is not None:
        _want(row_index, "row_index", dtype=torch.int32, device=dev)
        if row_index.dim() != 1:
            raise ValueError("row_index must be 1-D")
        M = row_index.shape[0]
    else:
        M = n_src
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    ld_out = _rows_view(out, "out", d, dev)
    if out.shape[0] != M:
        raise ValueError(f"out has {out.shape[0]} rows, expected {M}")
    return M, d, dev, (ctypes.c_int64 * 3)(*ld), n_src, out, ld_out


def fuse_rows(h_low, h_mid, h_high, norm, eps, gammas, betas, W: torch.Tensor, bias: Optional[torch.Tensor],
              row_index: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """eagle31_fuse_rows: as fuse(), token m reading row row_index[m] (or m)
    of the state views, which (like out) may have any row stride."""
    M, d, dev, ld, n_src, out, ld_out = _row_args(h_low, h_mid, h_high, row_index, out)
    _want(W, "W", shape=(3 * d, d), device=dev)
    if bias is not None:
        _want(bias, "bias", shape=(d,), device=dev)
    g = _vec3(gammas, "gammas", d, dev)
    b = _vec3(betas, "betas", d, dev)
    st = lib().eagle31_fuse_rows(_ptr(h_low), _ptr(h_mid), _ptr(h_high), ld, _ptr(row_index), n_src, M, d,
                                 norm_kind(norm), float(eps), g[0] if g else None, b[0] if b else None, _ptr(W),
                                 _ptr(bias), _ptr(out), ld_out, _stream(h_low))
    check("eagle31_fuse_rows", st)
    return out


def fuse_folded_rows(h_low, h_mid, h_high, norm, eps, w_folded: torch.Tensor, u: torch.Tensor, c: torch.Tensor,
                     row_index: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """eagle31_fuse_folded_rows: as fuse_folded(), token m reading row
    row_index[m] (or m) of the state views; any row strides."""
    M, d, dev, ld, n_src, out, ld_out = _row_args(h_low, h_mid, h_high, row_index, out)
    _want(w_folded, "w_folded", shape=folded_shape(d), device=dev)
    _want(u, "u", dtype=torch.float32, shape=(3, d), device=dev)
    _want(c, "c", dtype=torch.float32, shape=(d,), device=dev)
    st = lib().eagle31_fuse_folded_rows(_ptr(h_low), _ptr(h_mid), _ptr(h_high), ld, _ptr(row_index), n_src, M, d,
                                        norm_kind(norm), float(eps), _ptr(w_folded), _ptr(u), _ptr(c), _ptr(out),
                                        ld_out, _stream(h_low))
    check("eagle31_fuse_folded_rows", st)
    return out


def fuse_folded_noalloc(h_low, h_mid, h_high, norm, eps, w_folded: torch.Tensor, u: torch.Tensor, c: torch.Tensor,
                        out: torch.Tensor) -> torch.Tensor:
    """eagle31_fuse_folded_noalloc: the folded step on the library's fixed
    scratch array.  `out` must be given: nothing is allocated here either."""
    M, d, dev = _states(h_low, h_mid, h_high)
    _want(w_folded, "w_folded", shape=folded_shape(d), device=dev)
    _want(u, "u", dtype=torch.float32, shape=(3, d), device=dev)
    _want(c, "c", dtype=torch.float32, shape=(d,), device=dev)
    _want(out, "out", shape=(M, d), device=dev)
    st = lib().eagle31_fuse_folded_noalloc(_ptr(h_low), _ptr(h_mid), _ptr(h_high), M, d, norm_kind(norm), float(eps),
                                           _ptr(w_folded), _ptr(u), _ptr(c), _ptr(out), _stream(h_low))
    check("eagle31_fuse_folded_noalloc", st)
    return out


def noalloc_scratch_bytes() -> int:
    return int(lib().eagle31_noalloc_scratch_bytes())


def row_stats(h_low, h_mid, h_high, norm, eps):
    """eagle31_row_stats: returns (mu [3, M], rstd [3, M]) float32."""
    M, d, dev = _states(h_low, h_mid, h_high)
    mu = torch.empty((3, M), dtype=torch.float32, device=dev)
    rstd = torch.empty((3, M), dtype=torch.float32, device=dev)
    st = lib().eagle31_row_stats(_ptr(h_low), _ptr(h_mid), _ptr(h_high), M, d, norm_kind(norm), float(eps),
                                 _ptr(mu), _ptr(rstd), _stream(h_low))
    check("eagle31_row_stats", st)
    return mu, rstd


def norm_output(x, norm, eps, gamma=None, beta=None, out=None):
    """eagle31_norm_output: row norm of the drafter's output hidden state x
    [M, d] bf16 (post-norm feedback).  out=x normalises in place."""
    _want(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [M, d]")
    M, d = x.shape
    if gamma is not None:
        _want(gamma, "gamma", shape=(d,), device=x.device)
    if beta is not None:
        _want(beta, "beta", shape=(d,), device=x.device)
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=x.device)
    _want(out, "out", shape=(M, d), device=x.device)
    st = lib().eagle31_norm_output(_ptr(x), M, d, norm_kind(norm), float(eps), _ptr(gamma), _ptr(beta), _ptr(out),
                                   _stream(x))
    check("eagle31_norm_output", st)
    return out


def embed_concat(tokens, embed, fused, out=None, bad_count=None):
    """eagle31_embed_concat: [embed[tokens[m]] | fused[m]] per row -> bf16
    [M, 2d].  tokens int32 [M]; bad_count: optional int32 [1] device tensor
    that counts token ids outside the table (the caller zeroes it).  With
    fused None only the embedding half of out is written (out required)."""
    if (not isinstance(tokens, torch.Tensor) or tokens.dtype != torch.int32 or tokens.dim() != 1 or not tokens.is_cuda
            or not tokens.is_contiguous()):
        raise TypeError("tokens must be a contiguous 1-d int32 tensor on a GPU")
    _want(embed, "embed", device=tokens.device)
    if embed.dim() != 2:
        raise ValueError("embed must be [vocab, d]")
    vocab, d = embed.shape
    M = tokens.shape[0]
    if fused is not None:
        _want(fused, "fused", shape=(M, d), device=tokens.device)
    elif out is None:
        raise ValueError("without fused, out must be given (its right half is left as it is)")
    if out is None:
        out = torch.empty((M, 2 * d), dtype=torch.bfloat16, device=tokens.device)
    _want(out, "out", shape=(M, 2 * d), device=tokens.device)
    if bad_count is not None and (bad_count.dtype != torch.int32 or bad_count.numel() != 1 or not bad_count.is_cuda):
        raise TypeError("bad_count must be a one-element int32 tensor on a GPU")
    st = lib().eagle31_embed_concat(_ptr(tokens), M, d, vocab, _ptr(embed), _ptr(fused), _ptr(out), _ptr(bad_count),
                                    _stream(out))
    check("eagle31_embed_concat", st)
    return out


def verify_accept(p: torch.Tensor, q: torch.Tensor, draft: torch.Tensor, u_acc: torch.Tensor, u_res: torch.Tensor,
                  n_accepted: Optional[torch.Tensor] = None, next_token: Optional[torch.Tensor] = None):
    """eagle31_verify_accept: p [B, N, V], q [B, N+1, V] float32, draft [B, N]
    int32, u_acc [B, N], u_res [B] float32 -> (n_accepted [B], next_token [B]) int32."""
    if p.dim() != 3:
        raise ValueError("p must be [B, N, V]")
    B, N, V = p.shape
    dev = p.device
    _want(p, "p", dtype=torch.float32, device=dev)
    _want(q, "q", dtype=torch.float32, shape=(B, N + 1, V), device=dev)
    _want(draft, "draft", dtype=torch.int32, shape=(B, N), device=dev)
    _want(u_acc, "u_acc", dtype=torch.float32, shape=(B, N), device=dev)
    _want(u_res, "u_res", dtype=torch.float32, shape=(B,), device=dev)
    if n_accepted is None:
        n_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(B, dtype=torch.int32, device=dev)
    _want(n_accepted, "n_accepted", dtype=torch.int32, shape=(B,), device=dev)
    _want(next_token, "next_token", dtype=torch.int32, shape=(B,), device=dev)
    st = lib().eagle31_verify_accept(_ptr(p), _ptr(q), _ptr(draft), _ptr(u_acc), _ptr(u_res), B, N, V,
                                     _ptr(n_accepted), _ptr(next_token), _stream(p))
    check("eagle31_verify_accept", st)
    return n_accepted, next_token


def verify_chunking(B: int, N: int, V: int):
    """eagle31_verify_chunking: (chunks per row, tokens per chunk) of eagle31_verify_accept."""
    import ctypes
    c = ctypes.c_int32(0)
    t = ctypes.c_int32(0)
    check("eagle31_verify_chunking", lib().eagle31_verify_chunking(B, N, V, ctypes.byref(c), ctypes.byref(t)))
    return c.value, t.value


def release() -> None:
    check("eagle31_release", lib().eagle31_release())


def debug_stats_recompute(on: bool) -> None:
    """Test hook: the folded decode kernel's statistics readers recompute the
    rows instead of waiting for the published records (same result)."""
    check("eagle31_debug_stats_recompute", lib().eagle31_debug_stats_recompute(1 if on else 0))


def debug_fail_workspace_zero(on: bool) -> None:
    """Test hook: the counter zeroing of a new library-owned workspace reports
    a launch failure (and the buffer is not kept)."""
    check("eagle31_debug_fail_workspace_zero", lib().eagle31_debug_fail_workspace_zero(1 if on else 0))
