"""fp64 CPU oracle for the per-token mHC residual-mixing path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``mhc_hyper_connection_proj_amd``) and never imports it.

The arithmetic lives in ``mhc_oracle.c`` (plain C, double precision, one token at
a time).  This module only loads it, converts storage types exactly to float64,
and rounds each operation's outputs once to their storage type: bf16 with
round-to-nearest-even straight from float64, or float32.

Sources, cited per function: the Megatron Core "core.fusions.fused_mhc_kernels"
API page (the four fused operations and their torch reference signatures), the
rwkv-ops 0.6.1 ``mhu_ffi.cu`` diff page (FFI sections for Sinkhorn, stream
aggregate, post-op and pre-op) and RL-Kernel pull request #383 (RMS backward
zero-row guard, three segment gains).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mhc_oracle.c")
_LIB = os.path.join(_HERE, "libmhc_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
_i32 = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
             "-shared", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.mhc_oracle_proj_rms_h.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp, _dp, ctypes.c_double,
                                              _dp, _dp, _dp, _dp, _dp, _dp]
        lib.mhc_oracle_sinkhorn_fwd.argtypes = [_i64, _i32, _dp, _i32, ctypes.c_double, _dp]
        lib.mhc_oracle_sinkhorn_bwd.argtypes = [_i64, _i32, _dp, _dp, _i32, ctypes.c_double, _dp]
        lib.mhc_oracle_h_aggregate_fwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp]
        lib.mhc_oracle_h_aggregate_bwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp, _dp, _dp]
        lib.mhc_oracle_h_post_bda_fwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.mhc_oracle_h_post_bda_bwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp, _dp, _dp, _dp,
                                                  _dp, _dp, _dp, _dp, _dp]
        lib.mhc_oracle_proj_rms_h_bwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp, _dp, ctypes.c_double,
                                                  _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.mhc_oracle_stream_mix_fwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp]
        lib.mhc_oracle_stream_mix_bwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp, _dp, _dp]
        lib.mhc_oracle_stream_distribute_fwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp]
        lib.mhc_oracle_stream_distribute_bwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp, _dp, _dp]
        lib.mhc_oracle_h_aggregate_static_fwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp]
        lib.mhc_oracle_h_aggregate_static_bwd.argtypes = [_i64, _i32, _i64, _dp, _dp, _dp, _dp, _dp]
        lib.mhc_oracle_rmsnorm_fwd.argtypes = [_i64, _i64, _dp, _dp, ctypes.c_double, _dp, _dp]
        lib.mhc_oracle_rmsnorm_bwd.argtypes = [_i64, _i64, _dp, _dp, _dp, ctypes.c_double, _dp, _dp]
        for f in ("mhc_oracle_proj_rms_h", "mhc_oracle_sinkhorn_fwd", "mhc_oracle_sinkhorn_bwd",
                  "mhc_oracle_h_aggregate_fwd", "mhc_oracle_h_aggregate_bwd",
                  "mhc_oracle_h_post_bda_fwd", "mhc_oracle_h_post_bda_bwd",
                  "mhc_oracle_proj_rms_h_bwd", "mhc_oracle_stream_mix_fwd", "mhc_oracle_stream_mix_bwd",
                  "mhc_oracle_stream_distribute_fwd", "mhc_oracle_stream_distribute_bwd",
                  "mhc_oracle_h_aggregate_static_fwd", "mhc_oracle_h_aggregate_static_bwd",
                  "mhc_oracle_rmsnorm_fwd", "mhc_oracle_rmsnorm_bwd"):
            getattr(lib, f).restype = None
        _lib_handle = lib
    return _lib_handle


# --------------------------------------------------------------------------
# exact storage conversions
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns with one round-to-nearest-even step.

    bf16 keeps 8 significant bits with fp32's exponent range, so the spacing of
    representable values around v (with v = m * 2**e, 0.5 <= |m| < 1) is
    2**(e-8), floored at the subnormal spacing 2**-133.  Scaling by a power of
    two is exact and numpy's rint rounds half to even.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.maximum(e.astype(np.int64) - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)
    f = r.astype(np.float32)  # exact: r already has <= 8 significant bits
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def round_f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> the float64 value of its bf16 rounding."""
    return bf16_bits_to_f64(round_f64_to_bf16_bits(v))


def round_f64_to_f32(v: np.ndarray) -> np.ndarray:
    """float64 -> float32 (IEEE round-to-nearest-even) -> float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 results once to the storage type ('bf16' or 'f32'), returned as float64."""
    if dtype == "bf16":
        return round_f64_to_bf16(v)
    if dtype == "f32":
        return round_f64_to_f32(v)
    raise ValueError(dtype)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


# --------------------------------------------------------------------------
# single operations (float64 in, float64 out, no rounding)
# --------------------------------------------------------------------------
@dataclass
class ProjOut:
    H_pre: np.ndarray   # [N, n]
    H_post: np.ndarray  # [N, n]
    L: np.ndarray       # [N, n, n] Sinkhorn logits
    r: np.ndarray       # [N]
    q: np.ndarray       # [N]
    z: np.ndarray       # [N, J] pre-gain projection times r


def proj_rms_h(X, W, alpha=None, hbias=None, eps_rms=1e-6) -> ProjOut:
    """F1: projection + RMS + compute_h (Megatron ``_torch_proj_rms_compute_h``).

    X: [N, n, C]; W: [n*C, n*n+2n]; alpha: [3] (pre, post, res gains), default
    ones; hbias: [n*n+2n], default zeros.
    """
    X = _f64(X)
    N, n, C = X.shape
    J = n * n + 2 * n
    W = _f64(W).reshape(n * C, J)
    alpha = _f64(np.ones(3) if alpha is None else alpha)
    hbias = _f64(np.zeros(J) if hbias is None else hbias)
    H_pre = np.empty((N, n)); H_post = np.empty((N, n)); L = np.empty((N, n, n))
    r = np.empty(N); q = np.empty(N); z = np.empty((N, J))
    _lib().mhc_oracle_proj_rms_h(N, n, C, _p(X), _p(W), _p(alpha), _p(hbias), float(eps_rms),
                                 _p(H_pre), _p(H_post), _p(L), _p(r), _p(q), _p(z))
    return ProjOut(H_pre, H_post, L, r, q, z)


def sinkhorn_fwd(L, iters=20, eps=1e-6) -> np.ndarray:
    """F2: Sinkhorn-Knopp on exp(L), row pass then column pass per iteration.  L: [..., n, n]."""
    L = _f64(L)
    n = L.shape[-1]
    count = L.size // (n * n)
    H = np.empty_like(L)
    _lib().mhc_oracle_sinkhorn_fwd(count, n, _p(L), int(iters), float(eps), _p(H))
    return H


def sinkhorn_bwd(dH, L, iters=20, eps=1e-6) -> np.ndarray:
    """B2: exact reverse mode of the unrolled F2 map.  Returns dL with L's shape."""
    L = _f64(L)
    dH = _f64(dH).reshape(L.shape)
    n = L.shape[-1]
    count = L.size // (n * n)
    dL = np.empty_like(L)
    _lib().mhc_oracle_sinkhorn_bwd(count, n, _p(dH), _p(L), int(iters), float(eps), _p(dL))
    return dL


def h_aggregate_fwd(X, H_pre) -> np.ndarray:
    """F3: agg[t, c] = sum_i H_pre[t, i] X[t, i, c]."""
    X = _f64(X); H_pre = _f64(H_pre)
    N, n, C = X.shape
    agg = np.empty((N, C))
    _lib().mhc_oracle_h_aggregate_fwd(N, n, C, _p(X), _p(H_pre), _p(agg))
    return agg


def h_aggregate_bwd(g, X, H_pre):
    """B3: returns (dX [N,n,C], dH_pre [N,n])."""
    X = _f64(X); H_pre = _f64(H_pre); g = _f64(g)
    N, n, C = X.shape
    dX = np.empty((N, n, C)); dH = np.empty((N, n))
    _lib().mhc_oracle_h_aggregate_bwd(N, n, C, _p(g), _p(X), _p(H_pre), _p(dX), _p(dH))
    return dX, dH


def h_post_bda_fwd(X, H_res, H_post, x, bias=None) -> np.ndarray:
    """F4: out[t,i,c] = sum_j H_res[t,j,i] X[t,j,c] + H_post[t,i] (x[t,c] + bias[c])."""
    X = _f64(X); H_res = _f64(H_res); H_post = _f64(H_post); x = _f64(x)
    N, n, C = X.shape
    b = _f64(bias) if bias is not None else None
    out = np.empty((N, n, C))
    _lib().mhc_oracle_h_post_bda_fwd(N, n, C, _p(X), _p(H_res), _p(H_post), _p(x),
                                     _p(b) if b is not None else None, _p(out))
    return out


def h_post_bda_bwd(G, X, H_res, H_post, x, bias=None):
    """B4: returns (dX, dH_res, dH_post, dx, dbias-or-None)."""
    G = _f64(G); X = _f64(X); H_res = _f64(H_res); H_post = _f64(H_post); x = _f64(x)
    N, n, C = X.shape
    b = _f64(bias) if bias is not None else None
    dX = np.empty((N, n, C)); dHr = np.empty((N, n, n)); dHp = np.empty((N, n))
    dx = np.empty((N, C)); db = np.empty(C) if b is not None else None
    _lib().mhc_oracle_h_post_bda_bwd(N, n, C, _p(G), _p(X), _p(H_res), _p(H_post), _p(x),
                                     _p(b) if b is not None else None, _p(dX), _p(dHr), _p(dHp),
                                     _p(dx), _p(db) if db is not None else None)
    return dX, dHr, dHp, dx, db


def stream_mix_fwd(X, M) -> np.ndarray:
    """F5: out[t,i,c] = sum_j M[t,j,i] X[t,j,c] (rwkv-ops Stream Mix FFI)."""
    X = _f64(X); M = _f64(M)
    N, n, C = X.shape
    out = np.empty((N, n, C))
    _lib().mhc_oracle_stream_mix_fwd(N, n, C, _p(X), _p(M), _p(out))
    return out


def stream_mix_bwd(G, X, M):
    """B5: returns (dX [N,n,C], dM [N,n,n])."""
    G = _f64(G); X = _f64(X); M = _f64(M)
    N, n, C = X.shape
    dX = np.empty((N, n, C)); dM = np.empty((N, n, n))
    _lib().mhc_oracle_stream_mix_bwd(N, n, C, _p(G), _p(X), _p(M), _p(dX), _p(dM))
    return dX, dM


def stream_distribute_fwd(x, H_post) -> np.ndarray:
    """F6: out[t,i,c] = H_post[t,i] x[t,c] (rwkv-ops Stream Distribute FFI)."""
    x = _f64(x); H_post = _f64(H_post)
    (N, C), n = x.shape, H_post.shape[1]
    out = np.empty((N, n, C))
    _lib().mhc_oracle_stream_distribute_fwd(N, n, C, _p(x), _p(H_post), _p(out))
    return out


def stream_distribute_bwd(G, x, H_post):
    """B6: returns (dx [N,C], dH_post [N,n])."""
    G = _f64(G); x = _f64(x); H_post = _f64(H_post)
    (N, C), n = x.shape, H_post.shape[1]
    dx = np.empty((N, C)); dH = np.empty((N, n))
    _lib().mhc_oracle_stream_distribute_bwd(N, n, C, _p(G), _p(x), _p(H_post), _p(dx), _p(dH))
    return dx, dH


def h_aggregate_static_fwd(X, H_pre) -> np.ndarray:
    """F3s: agg[t, c] = sum_i H_pre[i] X[t, i, c], one H_pre row [n] for all tokens."""
    X = _f64(X); H_pre = _f64(H_pre)
    N, n, C = X.shape
    agg = np.empty((N, C))
    _lib().mhc_oracle_h_aggregate_static_fwd(N, n, C, _p(X), _p(H_pre), _p(agg))
    return agg


def h_aggregate_static_bwd(g, X, H_pre):
    """B3s: returns (dX [N,n,C], dH_pre [n]) with dH_pre summed over tokens."""
    X = _f64(X); H_pre = _f64(H_pre); g = _f64(g)
    N, n, C = X.shape
    dX = np.empty((N, n, C)); dH = np.empty(n)
    _lib().mhc_oracle_h_aggregate_static_bwd(N, n, C, _p(g), _p(X), _p(H_pre), _p(dX), _p(dH))
    return dX, dH


def rmsnorm_fwd(x, gamma=None, eps=1e-6):
    """F7: y[t,c] = gamma[c] x[t,c] / (sqrt(mean_c x[t,c]^2) + eps) (rwkv-ops RMSNorm FFI; gain
    per RL-Kernel's rmsnorm_residual).  gamma None = weightless.  Returns (y [N,C], r [N])."""
    x = _f64(x)
    N, C = x.shape
    g = _f64(gamma) if gamma is not None else None
    y = np.empty((N, C)); r = np.empty(N)
    _lib().mhc_oracle_rmsnorm_fwd(N, C, _p(x), _p(g) if g is not None else None, float(eps), _p(y), _p(r))
    return y, r


def rmsnorm_bwd(dy, x, gamma=None, eps=1e-6):
    """B7: returns (dx [N,C], dgamma [C] summed over tokens, or None when gamma is None)."""
    x = _f64(x); dy = _f64(dy)
    N, C = x.shape
    g = _f64(gamma) if gamma is not None else None
    dx = np.empty((N, C)); dg = np.empty(C) if g is not None else None
    _lib().mhc_oracle_rmsnorm_bwd(N, C, _p(dy), _p(x), _p(g) if g is not None else None, float(eps),
                                  _p(dx), _p(dg) if dg is not None else None)
    return dx, dg


def proj_rms_h_bwd(X, W, dH_pre, dH_post, dL, alpha=None, hbias=None, eps_rms=1e-6):
    """B1: returns (dX [N,n,C] (this op's own term), dW [K,J], dalpha [3], dhbias [J])."""
    X = _f64(X)
    N, n, C = X.shape
    J = n * n + 2 * n
    W = _f64(W).reshape(n * C, J)
    alpha = _f64(np.ones(3) if alpha is None else alpha)
    hbias = _f64(np.zeros(J) if hbias is None else hbias)
    dH_pre = _f64(dH_pre); dH_post = _f64(dH_post); dL = _f64(dL)
    dX = np.empty((N, n, C)); dW = np.empty((n * C, J)); da = np.empty(3); db = np.empty(J)
    _lib().mhc_oracle_proj_rms_h_bwd(N, n, C, _p(X), _p(W), _p(alpha), _p(hbias), float(eps_rms),
                                     _p(dH_pre), _p(dH_post), _p(dL), _p(dX), _p(dW), _p(da), _p(db))
    return dX, dW, da, db


# --------------------------------------------------------------------------
# compositions (the fused passes): still plain sequences of the ops above
# --------------------------------------------------------------------------
def pre_fwd(X, W, alpha=None, hbias=None, eps_rms=1e-6, iters=20, eps=1e-6):
    """Pre pass forward: F1 -> F2 on the logits -> F3 with H_pre.  All float64.

    Returns dict with H_pre, H_post, H_res, L, r, q, z, agg (agg unrounded).
    """
    p = proj_rms_h(X, W, alpha, hbias, eps_rms)
    H_res = sinkhorn_fwd(p.L, iters, eps)
    agg = h_aggregate_fwd(X, p.H_pre)
    return dict(H_pre=p.H_pre, H_post=p.H_post, H_res=H_res, L=p.L, r=p.r, q=p.q, z=p.z, agg=agg)


def pre_bwd(g, dH_post, dH_res, X, W, alpha=None, hbias=None, eps_rms=1e-6, iters=20, eps=1e-6):
    """Pre pass backward: B3 (dH_pre, dX term) + B2 (dL) + B1, summed dX.

    g = gradient of the aggregated stream [N, C]; dH_post [N, n]; dH_res [N, n, n].
    Returns dict with dX (sum of the aggregate and projection terms, unrounded),
    dW, dalpha, dhbias, dH_pre, dL.
    """
    p = proj_rms_h(X, W, alpha, hbias, eps_rms)
    dX_agg, dH_pre = h_aggregate_bwd(g, X, p.H_pre)
    dL = sinkhorn_bwd(dH_res, p.L, iters, eps)
    dX_proj, dW, da, db = proj_rms_h_bwd(X, W, dH_pre, dH_post, dL, alpha, hbias, eps_rms)
    return dict(dX=dX_agg + dX_proj, dW=dW, dalpha=da, dhbias=db, dH_pre=dH_pre, dL=dL)
