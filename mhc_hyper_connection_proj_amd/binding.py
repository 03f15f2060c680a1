"""Torch-facing binding of libmhc: one function per C entry point, same names.

Each function checks dtypes/shapes/contiguity, allocates the outputs and the
workspace with torch.empty on the input's device, and calls the C ABI on the
current HIP stream.  No arithmetic happens here.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import MHC_BF16, MHC_F32, call


def n_outputs(n: int) -> int:
    """J = n*n + 2n controller outputs for n streams."""
    return n * n + 2 * n


def saved_stride(n: int) -> int:
    """Row stride of the saved forward state (mhc_saved_stride)."""
    return int(_lib.lib().mhc_saved_stride(n))


def _act(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MHC_BF16
    if t.dtype == torch.float32:
        return MHC_F32
    raise TypeError(f"activation dtype must be bfloat16 or float32, got {t.dtype}")


def _need(t: torch.Tensor | None, name: str, dtype=None, numel=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def _p(t):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ws(nbytes: int, dev):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=dev), nbytes


def _dims(X: torch.Tensor):
    if X.dim() < 2:
        raise ValueError("residual must be [..., n, C]")
    n, C = X.shape[-2], X.shape[-1]
    return X.numel() // (n * C) if n * C else 0, n, C


f32 = torch.float32


def mhc_proj_rms_h(X, W, alpha=None, hbias=None, rms_eps=1e-6, _entry="mhc_proj_rms_h"):
    """Projection + RMS + compute_h.  Returns (H_pre, H_post, H_res_logits, saved)."""
    N, n, C = _dims(X)
    J = n_outputs(n)
    act = _act(X)
    _need(X, "X"); _need(W, "W", f32, n * C * J); _need(alpha, "alpha", f32, 3); _need(hbias, "hbias", f32, J)
    lead = X.shape[:-2]
    d = X.device
    H_pre = torch.empty(*lead, n, dtype=f32, device=d)
    H_post = torch.empty(*lead, n, dtype=f32, device=d)
    L = torch.empty(*lead, n, n, dtype=f32, device=d)
    saved = torch.empty(*lead, saved_stride(n), dtype=f32, device=d)
    ws, wsb = _ws(_lib.lib().mhc_proj_rms_h_workspace_size(N, n, C, act), d)
    call(_entry, _stream(X), N, n, C, act, _p(X), _p(W), _p(alpha), _p(hbias), rms_eps,
         _p(H_pre), _p(H_post), _p(L), _p(saved), _p(ws), wsb)
    return H_pre, H_post, L, saved


def mhc_proj_rms_h_fma(X, W, alpha=None, hbias=None, rms_eps=1e-6):
    """mhc_proj_rms_h with x @ W as fp32 FMAs on the vector ALUs (the comparison point of the MFMA form;
    n = 4, bf16).  Returns (H_pre, H_post, H_res_logits, saved)."""
    return mhc_proj_rms_h(X, W, alpha, hbias, rms_eps, _entry="mhc_proj_rms_h_fma")


def mhc_proj_rms_h_bwd(X, W, saved, H_pre, H_post, dH_pre, dH_post, dH_res_logits, alpha=None,
                       dX=None, accumulate_dX=False, want_dW=True, want_dalpha=True, want_dhbias=True):
    """Projection backward.  Returns (dX, dW, dalpha, dhbias); skipped grads are None."""
    N, n, C = _dims(X)
    J = n_outputs(n)
    act = _act(X)
    for t, nm, ne in ((saved, "saved", N * saved_stride(n)), (H_pre, "H_pre", N * n), (H_post, "H_post", N * n),
                      (dH_pre, "dH_pre", N * n), (dH_post, "dH_post", N * n),
                      (dH_res_logits, "dH_res_logits", N * n * n)):
        _need(t, nm, f32, ne)
    _need(X, "X"); _need(W, "W", f32, n * C * J); _need(alpha, "alpha", f32, 3)
    d = X.device
    if dX is None:
        if accumulate_dX:
            raise ValueError("accumulate_dX needs dX")
        dX = torch.empty_like(X)
    _need(dX, "dX", X.dtype, X.numel())
    dW = torch.empty(n * C, J, dtype=f32, device=d) if want_dW else None
    da = torch.empty(3, dtype=f32, device=d) if want_dalpha else None
    db = torch.empty(J, dtype=f32, device=d) if want_dhbias else None
    ws, wsb = _ws(_lib.lib().mhc_proj_rms_h_bwd_workspace_size(N, n, C, act), d)
    call("mhc_proj_rms_h_bwd", _stream(X), N, n, C, act, _p(X), _p(W), _p(alpha), _p(saved), _p(H_pre),
         _p(H_post), _p(dH_pre), _p(dH_post), _p(dH_res_logits), _p(dX), int(accumulate_dX), _p(dW),
         _p(da), _p(db), _p(ws), wsb)
    return dX, dW, da, db


def mhc_sinkhorn_fwd(logits, iters=20, eps=1e-6):
    """Sinkhorn-Knopp projection of [..., n, n] fp32 logits."""
    n = logits.shape[-1]
    _need(logits, "logits", f32)
    count = logits.numel() // (n * n) if n else 0
    H = torch.empty_like(logits)
    call("mhc_sinkhorn_fwd", _stream(logits), count, n, _p(logits), _p(H), iters, eps)
    return H


def mhc_sinkhorn_bwd(dH_res, logits, iters=20, eps=1e-6):
    """Gradient of the Sinkhorn projection with respect to the logits."""
    n = logits.shape[-1]
    _need(logits, "logits", f32); _need(dH_res, "dH_res", f32, logits.numel())
    count = logits.numel() // (n * n) if n else 0
    dL = torch.empty_like(logits)
    call("mhc_sinkhorn_bwd", _stream(logits), count, n, _p(dH_res), _p(logits), _p(dL), iters, eps)
    return dL


def mhc_h_aggregate_fwd(X, H_pre):
    N, n, C = _dims(X)
    act = _act(X)
    _need(X, "X"); _need(H_pre, "H_pre", f32, N * n)
    out = torch.empty(*X.shape[:-2], C, dtype=X.dtype, device=X.device)
    call("mhc_h_aggregate_fwd", _stream(X), N, n, C, act, _p(X), _p(H_pre), _p(out))
    return out


def mhc_h_aggregate_bwd(g, X, H_pre, dX=None, accumulate_dX=False):
    """Returns (dX, dH_pre)."""
    N, n, C = _dims(X)
    act = _act(X)
    _need(X, "X"); _need(g, "g", X.dtype, N * C); _need(H_pre, "H_pre", f32, N * n)
    if dX is None:
        if accumulate_dX:
            raise ValueError("accumulate_dX needs dX")
        dX = torch.empty_like(X)
    _need(dX, "dX", X.dtype, X.numel())
    dH = torch.empty(*X.shape[:-2], n, dtype=f32, device=X.device)
    call("mhc_h_aggregate_bwd", _stream(X), N, n, C, act, _p(g), _p(X), _p(H_pre), _p(dX),
         int(accumulate_dX), _p(dH))
    return dX, dH


def mhc_h_aggregate_static_fwd(X, H_pre):
    """h_aggregate with one H_pre row [n] for all tokens."""
    N, n, C = _dims(X)
    act = _act(X)
    _need(X, "X"); _need(H_pre, "H_pre", f32, n)
    out = torch.empty(*X.shape[:-2], C, dtype=X.dtype, device=X.device)
    call("mhc_h_aggregate_static_fwd", _stream(X), N, n, C, act, _p(X), _p(H_pre), _p(out))
    return out


def mhc_h_aggregate_static_bwd(g, X, H_pre, dX=None, accumulate_dX=False):
    """Returns (dX, dH_pre [n]) for one shared H_pre row; dH_pre is summed over tokens."""
    N, n, C = _dims(X)
    act = _act(X)
    _need(X, "X"); _need(g, "g", X.dtype, N * C); _need(H_pre, "H_pre", f32, n)
    if dX is None:
        if accumulate_dX:
            raise ValueError("accumulate_dX needs dX")
        dX = torch.empty_like(X)
    _need(dX, "dX", X.dtype, X.numel())
    dH = torch.empty(n, dtype=f32, device=X.device)
    ws, wsb = _ws(_lib.lib().mhc_h_aggregate_static_bwd_workspace_size(N, n, C, act), X.device)
    call("mhc_h_aggregate_static_bwd", _stream(X), N, n, C, act, _p(g), _p(X), _p(H_pre), _p(dX),
         int(accumulate_dX), _p(dH), _p(ws), wsb)
    return dX, dH


def mhc_stream_mix_fwd(X, M):
    """out[i] = sum_j M[j][i] X[j] per token."""
    N, n, C = _dims(X)
    _need(X, "X"); _need(M, "M", f32, N * n * n)
    out = torch.empty_like(X)
    call("mhc_stream_mix_fwd", _stream(X), N, n, C, _act(X), _p(X), _p(M), _p(out))
    return out


def mhc_stream_mix_bwd(G, X, M):
    """Returns (dX, dM)."""
    N, n, C = _dims(X)
    _need(X, "X"); _need(G, "G", X.dtype, X.numel()); _need(M, "M", f32, N * n * n)
    dX = torch.empty_like(X)
    dM = torch.empty(*X.shape[:-2], n, n, dtype=f32, device=X.device)
    call("mhc_stream_mix_bwd", _stream(X), N, n, C, _act(X), _p(G), _p(X), _p(M), _p(dX), _p(dM))
    return dX, dM


def mhc_stream_distribute_fwd(x, H_post):
    """out[i] = H_post[i] x per token; x [..., C], H_post [..., n] -> [..., n, C]."""
    n, C = H_post.shape[-1], x.shape[-1]
    N = x.numel() // C if C else 0
    _need(x, "x"); _need(H_post, "H_post", f32, N * n)
    out = torch.empty(*x.shape[:-1], n, C, dtype=x.dtype, device=x.device)
    call("mhc_stream_distribute_fwd", _stream(x), N, n, C, _act(x), _p(x), _p(H_post), _p(out))
    return out


def mhc_stream_distribute_bwd(G, x, H_post):
    """Returns (dx, dH_post)."""
    n, C = H_post.shape[-1], x.shape[-1]
    N = x.numel() // C if C else 0
    _need(x, "x"); _need(G, "G", x.dtype, N * n * C); _need(H_post, "H_post", f32, N * n)
    dx = torch.empty_like(x)
    dH = torch.empty(*x.shape[:-1], n, dtype=f32, device=x.device)
    call("mhc_stream_distribute_bwd", _stream(x), N, n, C, _act(x), _p(G), _p(x), _p(H_post), _p(dx), _p(dH))
    return dx, dH


def mhc_h_post_bda_fwd(X, H_res, H_post, x, bias=None):
    N, n, C = _dims(X)
    act = _act(X)
    _need(X, "X"); _need(H_res, "H_res", f32, N * n * n); _need(H_post, "H_post", f32, N * n)
    _need(x, "x", X.dtype, N * C); _need(bias, "bias", X.dtype, C)
    out = torch.empty_like(X)
    call("mhc_h_post_bda_fwd", _stream(X), N, n, C, act, _p(X), _p(H_res), _p(H_post), _p(x), _p(bias), _p(out))
    return out


def mhc_h_post_bda_bwd(G, X, H_res, H_post, x, bias=None, want_dbias=True, want_dX=True):
    """Returns (dX-or-None, dH_res, dH_post, dx, dbias-or-None)."""
    N, n, C = _dims(X)
    act = _act(X)
    _need(X, "X"); _need(G, "G", X.dtype, X.numel()); _need(H_res, "H_res", f32, N * n * n)
    _need(H_post, "H_post", f32, N * n); _need(x, "x", X.dtype, N * C); _need(bias, "bias", X.dtype, C)
    d = X.device
    dX = torch.empty_like(X) if want_dX else None
    dHr = torch.empty(*X.shape[:-2], n, n, dtype=f32, device=d)
    dHp = torch.empty(*X.shape[:-2], n, dtype=f32, device=d)
    dx = torch.empty(*X.shape[:-2], C, dtype=X.dtype, device=d)
    db = torch.empty(C, dtype=X.dtype, device=d) if (bias is not None and want_dbias) else None
    ws, wsb = _ws(_lib.lib().mhc_h_post_bda_bwd_workspace_size(N, n, C, act, int(db is not None)), d)
    call("mhc_h_post_bda_bwd", _stream(X), N, n, C, act, _p(G), _p(X), _p(H_res), _p(H_post), _p(x), _p(bias),
         _p(dX), _p(dHr), _p(dHp), _p(dx), _p(db), _p(ws), wsb)
    return dX, dHr, dHp, dx, db


def mhc_pre_fwd(X, W, alpha=None, hbias=None, rms_eps=1e-6, iters=20, eps=1e-6):
    """Fused pre pass.  Returns dict(H_pre, H_post, H_res, H_res_logits, saved, agg)."""
    N, n, C = _dims(X)
    J = n_outputs(n)
    act = _act(X)
    _need(X, "X"); _need(W, "W", f32, n * C * J); _need(alpha, "alpha", f32, 3); _need(hbias, "hbias", f32, J)
    lead = X.shape[:-2]
    d = X.device
    o = dict(H_pre=torch.empty(*lead, n, dtype=f32, device=d), H_post=torch.empty(*lead, n, dtype=f32, device=d),
             H_res=torch.empty(*lead, n, n, dtype=f32, device=d),
             H_res_logits=torch.empty(*lead, n, n, dtype=f32, device=d),
             saved=torch.empty(*lead, saved_stride(n), dtype=f32, device=d),
             agg=torch.empty(*lead, C, dtype=X.dtype, device=d))
    ws, wsb = _ws(_lib.lib().mhc_pre_fwd_workspace_size(N, n, C, act), d)
    call("mhc_pre_fwd", _stream(X), N, n, C, act, _p(X), _p(W), _p(alpha), _p(hbias), rms_eps, iters, eps,
         _p(o["H_pre"]), _p(o["H_post"]), _p(o["H_res"]), _p(o["H_res_logits"]), _p(o["saved"]), _p(o["agg"]),
         _p(ws), wsb)
    return o


def _rows(x: torch.Tensor):
    if x.dim() < 1:
        raise ValueError("x must be [..., C]")
    C = x.shape[-1]
    return (x.numel() // C if C else 0), C


def mhc_rmsnorm_fwd(x, gamma=None, eps=1e-6):
    """RMSNorm of each row of x [..., C] with optional fp32 gain gamma [C]."""
    N, C = _rows(x)
    act = _act(x)
    _need(x, "x"); _need(gamma, "gamma", f32, C)
    y = torch.empty_like(x)
    call("mhc_rmsnorm_fwd", _stream(x), N, C, act, _p(x), _p(gamma), eps, _p(y))
    return y


def mhc_rmsnorm_bwd(dy, x, gamma=None, eps=1e-6, dx=None, accumulate_dx=False, want_dgamma=None):
    """Returns (dx, dgamma-or-None).  dgamma is produced when gamma is given (or want_dgamma=True).

    dx with accumulate_dx=True adds the norm's input gradient onto dx (the residual fork's own gradient).
    """
    N, C = _rows(x)
    act = _act(x)
    _need(x, "x"); _need(dy, "dy", x.dtype, x.numel()); _need(gamma, "gamma", f32, C)
    if dx is None:
        if accumulate_dx:
            raise ValueError("accumulate_dx needs dx")
        dx = torch.empty_like(x)
    _need(dx, "dx", x.dtype, x.numel())
    if want_dgamma is None:
        want_dgamma = gamma is not None
    dg = torch.empty(C, dtype=f32, device=x.device) if want_dgamma else None
    ws, wsb = _ws(_lib.lib().mhc_rmsnorm_bwd_workspace_size(N, C, act, int(want_dgamma)), x.device)
    call("mhc_rmsnorm_bwd", _stream(x), N, C, act, _p(dy), _p(x), _p(gamma), eps, _p(dx), int(accumulate_dx),
         _p(dg), _p(ws), wsb)
    return dx, dg


def mhc_pre_rmsnorm_fwd(X, W, gamma=None, alpha=None, hbias=None, rms_eps=1e-6, iters=20, eps=1e-6,
                        norm_eps=1e-6):
    """Fused pre pass with the norm epilogue.  Returns mhc_pre_fwd's dict plus 'normed' = RMSNorm(agg)."""
    N, n, C = _dims(X)
    J = n_outputs(n)
    act = _act(X)
    _need(X, "X"); _need(W, "W", f32, n * C * J); _need(alpha, "alpha", f32, 3); _need(hbias, "hbias", f32, J)
    _need(gamma, "gamma", f32, C)
    lead = X.shape[:-2]
    d = X.device
    o = dict(H_pre=torch.empty(*lead, n, dtype=f32, device=d), H_post=torch.empty(*lead, n, dtype=f32, device=d),
             H_res=torch.empty(*lead, n, n, dtype=f32, device=d),
             H_res_logits=torch.empty(*lead, n, n, dtype=f32, device=d),
             saved=torch.empty(*lead, saved_stride(n), dtype=f32, device=d),
             agg=torch.empty(*lead, C, dtype=X.dtype, device=d),
             normed=torch.empty(*lead, C, dtype=X.dtype, device=d))
    ws, wsb = _ws(_lib.lib().mhc_pre_fwd_workspace_size(N, n, C, act), d)
    call("mhc_pre_rmsnorm_fwd", _stream(X), N, n, C, act, _p(X), _p(W), _p(alpha), _p(hbias), rms_eps, iters,
         eps, _p(gamma), norm_eps, _p(o["H_pre"]), _p(o["H_post"]), _p(o["H_res"]), _p(o["H_res_logits"]),
         _p(o["saved"]), _p(o["agg"]), _p(o["normed"]), _p(ws), wsb)
    return o


def mhc_pre_bwd(g, dH_post, dH_res, X, W, saved, H_pre, H_post, H_res_logits, alpha=None, iters=20, eps=1e-6,
                dX=None, accumulate_dX=False, want_intermediates=False, post_G=None, post_H_res=None, want_dW=True):
    """Fused pre pass backward.  Returns dict(dX, dW, dalpha, dhbias[, dH_pre, dlogits]); dW is None
    when want_dW is False.

    post_G / post_H_res: the h_post_bda upstream gradient and H_res; when given,
    the h_post_bda dX term is added here (call mhc_h_post_bda_bwd with want_dX=False).
    """
    N, n, C = _dims(X)
    J = n_outputs(n)
    act = _act(X)
    _need(X, "X"); _need(g, "g", X.dtype, N * C); _need(dH_post, "dH_post", f32, N * n)
    _need(dH_res, "dH_res", f32, N * n * n); _need(W, "W", f32, n * C * J); _need(alpha, "alpha", f32, 3)
    _need(saved, "saved", f32, N * saved_stride(n)); _need(H_pre, "H_pre", f32, N * n)
    _need(H_post, "H_post", f32, N * n); _need(H_res_logits, "H_res_logits", f32, N * n * n)
    _need(post_G, "post_G", X.dtype, X.numel()); _need(post_H_res, "post_H_res", f32, N * n * n)
    d = X.device
    if dX is None:
        if accumulate_dX:
            raise ValueError("accumulate_dX needs dX")
        dX = torch.empty_like(X)
    _need(dX, "dX", X.dtype, X.numel())
    o = dict(dX=dX, dW=torch.empty(n * C, J, dtype=f32, device=d) if want_dW else None,
             dalpha=torch.empty(3, dtype=f32, device=d), dhbias=torch.empty(J, dtype=f32, device=d))
    if want_intermediates:
        o["dH_pre"] = torch.empty(*X.shape[:-2], n, dtype=f32, device=d)
        o["dlogits"] = torch.empty(*X.shape[:-2], n, n, dtype=f32, device=d)
    ws, wsb = _ws(_lib.lib().mhc_pre_bwd_workspace_size(N, n, C, act), d)
    call("mhc_pre_bwd", _stream(X), N, n, C, act, _p(g), _p(dH_post), _p(dH_res), _p(X), _p(W), _p(alpha),
         _p(saved), _p(H_pre), _p(H_post), _p(H_res_logits), iters, eps, _p(post_G), _p(post_H_res), _p(dX),
         int(accumulate_dX),
         _p(o["dW"]), _p(o["dalpha"]), _p(o["dhbias"]), _p(o.get("dH_pre")), _p(o.get("dlogits")),
         _p(ws), wsb)
    return o


def mhc_pre_rmsnorm_bwd(dy, agg, dH_post, dH_res, X, W, saved, H_pre, H_post, H_res_logits, gamma=None,
                        norm_eps=1e-6, g_fork=None, alpha=None, iters=20, eps=1e-6, dX=None, accumulate_dX=False,
                        post_G=None, post_H_res=None, want_dgamma=None, want_d_agg=False):
    """Fused pre pass backward with the norm's backward in front (the backward of mhc_pre_rmsnorm_fwd).
    Returns dict(dX, dW, dalpha, dhbias[, dgamma][, d_agg]).  g_fork: agg's own upstream gradient."""
    N, n, C = _dims(X)
    J = n_outputs(n)
    act = _act(X)
    _need(X, "X"); _need(dy, "dy", X.dtype, N * C); _need(agg, "agg", X.dtype, N * C)
    _need(gamma, "gamma", f32, C); _need(g_fork, "g_fork", X.dtype, N * C)
    _need(dH_post, "dH_post", f32, N * n); _need(dH_res, "dH_res", f32, N * n * n); _need(W, "W", f32, n * C * J)
    _need(alpha, "alpha", f32, 3); _need(saved, "saved", f32, N * saved_stride(n)); _need(H_pre, "H_pre", f32, N * n)
    _need(H_post, "H_post", f32, N * n); _need(H_res_logits, "H_res_logits", f32, N * n * n)
    _need(post_G, "post_G", X.dtype, X.numel()); _need(post_H_res, "post_H_res", f32, N * n * n)
    d = X.device
    if dX is None:
        if accumulate_dX:
            raise ValueError("accumulate_dX needs dX")
        dX = torch.empty_like(X)
    _need(dX, "dX", X.dtype, X.numel())
    if want_dgamma is None:
        want_dgamma = gamma is not None
    o = dict(dX=dX, dW=torch.empty(n * C, J, dtype=f32, device=d), dalpha=torch.empty(3, dtype=f32, device=d),
             dhbias=torch.empty(J, dtype=f32, device=d))
    if want_dgamma:
        o["dgamma"] = torch.empty(C, dtype=f32, device=d)
    if want_d_agg:
        o["d_agg"] = torch.empty(N, C, dtype=X.dtype, device=d)
    ws, wsb = _ws(_lib.lib().mhc_pre_rmsnorm_bwd_workspace_size(N, n, C, act, int(want_dgamma)), d)
    call("mhc_pre_rmsnorm_bwd", _stream(X), N, n, C, act, _p(dy), _p(agg), _p(gamma), norm_eps, _p(g_fork),
         _p(dH_post), _p(dH_res), _p(X), _p(W), _p(alpha), _p(saved), _p(H_pre), _p(H_post), _p(H_res_logits),
         iters, eps, _p(post_G), _p(post_H_res), _p(dX), int(accumulate_dX), _p(o["dW"]), _p(o["dalpha"]),
         _p(o["dhbias"]), _p(o.get("dgamma")), _p(o.get("d_agg")), _p(ws), wsb)
    return o
