"""Helpers for the GPU parity tests: host<->device transfer and tolerance rules.

Tolerances (stated by the benchmark spec for this path, applied element by element):
  * fp32 H tensors (H_pre, H_post, H_res, r): |g - o| <= 1e-5 |o|
  * fp32 quantities that cross zero (logits, z, gradients, dW, ...):
    |g - o| <= 1e-5 (|o| + rms(o)), i.e. 1e-5 relative to the tensor's scale
  * for both fp32 rules, an exact value below fp32's normal range (2^-126)
    is matched to within 2^-126: fp32 cannot hold it more precisely (the
    Sinkhorn gradient of a single stream, n = 1, is ~eps^(2 iters))
  * bf16 tensors: |g - o| <= 8e-3 |o| + 1e-5 rms(o), o being the oracle's fp64
    result rounded once to bf16 (8e-3 is one bf16 ulp; the small absolute
    term absorbs fp32 accumulation on cancelling sums).
  * sums over tokens (dW, dalpha, dhbias, dbias): the rule of their type plus
    1e-5 sum_t |o_t|, o_t being token t's own contribution from the oracle.
    Each token's contribution carries the per-token 1e-5 relative error, and
    the errors add across tokens; when the contributions cancel, the sum is
    far smaller than they are and a bound relative to the sum alone is not
    attainable in fp32.
"""
import os
import sys

import numpy as np
import torch

import oracle as O


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, act: str | None = None) -> torch.Tensor:
    """Host storage array -> CUDA tensor (uint16 bit patterns become bfloat16)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def h64(a) -> np.ndarray:
    """Storage array (bf16 bits or float) or tensor -> exact float64 numpy."""
    if isinstance(a, torch.Tensor):
        return a.detach().float().cpu().double().numpy()
    if a.dtype == np.uint16:
        return O.bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


DUMP_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out", "parity_dumps")


def _dump(name, g, o, bound):
    """On a parity failure, keep the compared tensors (gpu, oracle, bound) for offline reading."""
    try:
        os.makedirs(DUMP_DIR, exist_ok=True)
        safe = "".join(ch if ch.isalnum() else "_" for ch in name)
        path = os.path.join(DUMP_DIR, f"{safe}_{os.getpid()}.npz")
        np.savez_compressed(path, gpu=g, oracle=o, bound=np.broadcast_to(bound, np.shape(g)))
        return path
    except OSError:
        return None


def _report(name, g, o, bound):
    err = np.abs(g - o)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        path = _dump(name, g, o, bound)
        log(f"{name}: parity failure, tensors kept in {path}")
        raise AssertionError(
            f"{name}: {bad.sum()} of {bad.size} elements out of tolerance; worst at {i}: "
            f"gpu={g[i]!r} oracle={o[i]!r} err={err[i]:.3e} bound={bound[i] if np.ndim(bound) else bound:.3e}")


# fp32 holds no value below its normal range (2^-126) to relative precision:
# there an fp32 result may differ from the exact value by up to 2^-126.
FP32_TINY = 2.0 ** -126


def _fp32_floor(bound, o):
    return np.maximum(bound, np.where(np.abs(o) < FP32_TINY, FP32_TINY, 0.0))


def assert_rel(name, g, o, rtol=1e-5):
    g = h64(g); o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (name, g.shape, o.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    _report(name, g, o, _fp32_floor(rtol * np.abs(o), o))


def assert_mixed(name, g, o, rtol=1e-5):
    g = h64(g); o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (name, g.shape, o.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    rms = np.sqrt(np.mean(o * o)) if o.size else 0.0
    _report(name, g, o, _fp32_floor(rtol * (np.abs(o) + rms), o))


def assert_tokensum(name, g, o, abs_parts, act="f32"):
    """Sum over tokens: abs_parts = sum_t |o_t| (same shape as o), see the module rules."""
    g = h64(g); o = np.asarray(o, np.float64); s = np.asarray(abs_parts, np.float64)
    assert g.shape == o.shape == s.shape, (name, g.shape, o.shape, s.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    rms = np.sqrt(np.mean(o * o)) if o.size else 0.0
    if act == "bf16":
        ob = O.round_f64_to_bf16(o)
        _report(name, g, ob, 8e-3 * np.abs(ob) + 1e-5 * rms + 1e-5 * s)
    else:
        _report(name, g, o, 1e-5 * (np.abs(o) + rms) + 1e-5 * s)


def pre_bwd_abs_parts(g, dH_post, dH_res, X, W, *rest):
    """sum_t |contribution of token t| to dW, dalpha, dhbias (oracle, one token at a time)."""
    aW = aa = ab = 0.0
    for t in range(X.shape[0]):
        r = O.pre_bwd(g[t:t + 1], dH_post[t:t + 1], dH_res[t:t + 1], X[t:t + 1], W, *rest)
        aW = aW + np.abs(r["dW"]); aa = aa + np.abs(r["dalpha"]); ab = ab + np.abs(r["dhbias"])
    return aW, aa, ab


def proj_bwd_abs_parts(X, W, dH_pre, dH_post, dL, *rest):
    """As pre_bwd_abs_parts for the projection backward alone."""
    aW = aa = ab = 0.0
    for t in range(X.shape[0]):
        _, dW, da, db = O.proj_rms_h_bwd(X[t:t + 1], W, dH_pre[t:t + 1], dH_post[t:t + 1], dL[t:t + 1], *rest)
        aW = aW + np.abs(dW); aa = aa + np.abs(da); ab = ab + np.abs(db)
    return aW, aa, ab


def assert_act(name, g, o, act):
    """Activation-typed output: bf16 rule against the oracle rounded to bf16, fp32 mixed rule."""
    g = h64(g); o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (name, g.shape, o.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    if act == "bf16":
        ob = O.round_f64_to_bf16(o)
        rms = np.sqrt(np.mean(o * o)) if o.size else 0.0
        _report(name, g, ob, 8e-3 * np.abs(ob) + 1e-5 * rms)
    else:
        assert_mixed(name, g, o)
