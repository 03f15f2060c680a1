"""Helpers for the GPU parity tests: host<->device transfer and tolerance rules.

Tolerances (stated for this path, applied element by element):
  * fp32 H tensors (H_pre, H_post, H_res, r): |g - o| <= 1e-5 |o|
  * fp32 quantities that cross zero (logits, z, gradients, dW, ...):
    |g - o| <= 1e-5 (|o| + rms(o)), i.e. 1e-5 relative to the tensor's scale
  * for both fp32 rules, an exact value below fp32's normal range (2^-126)
    is matched to within 2^-126: fp32 cannot hold it more precisely (the
    Sinkhorn gradient of a single stream, n = 1, is ~eps^(2 iters))
  * bf16 tensors: |g - o| <= 8e-3 |o| + 1e-5 rms(o), o being the oracle's fp64
    result rounded once to bf16 (8e-3 is one bf16 ulp; the small absolute
    term absorbs fp32 accumulation on cancelling sums).
  * fp32 sums over tokens (dW, dalpha, dhbias, fp32 dbias, dgamma, shared-row
    dH_pre): the rule of their type plus (1e-5 + gamma_d) sum_t |o_t|, o_t
    being token t's own contribution from the oracle.  1e-5 sum_t |o_t|: each
    contribution is formed from per-token values that the per-token rules
    hold to 1e-5, and the errors of the contributions add.  gamma_d =
    d u / (1 - d u) (u = 2^-24) bounds the fp32 summation itself, d being the
    longest chain of rounded operations that a nonzero contribution takes
    through the kernel's fixed reduction tree (sum_depth).  bf16 sums over
    tokens (dbias) are held to the bf16 rule alone.
  * Sinkhorn gradients of n != 4 beyond 50 iterations: see sinkhorn_rtol.

The oracle is only ever fed seeded inputs or its own results (rounded to their storage type).
Where a GPU step's result depends on a GPU-computed upstream value (the fused H_res on the GPU's
logits, the normed output on the GPU's agg), the expected value is the oracle's own, and the GPU's
measured upstream deviation enters only the bound, carried through the step to first order.
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


U32 = 2.0 ** -24  # fp32 unit roundoff


def gamma_fp32(d: int) -> float:
    """gamma_d = d u / (1 - d u): relative bound on a value that passes through d rounded fp32 operations."""
    return d * U32 / (1.0 - d * U32)


def _cdiv(a, b):
    return -(-int(a) // int(b))


def _rup(a, b):
    return _cdiv(a, b) * b


def dxdw_token_block(N: int, C: int, n: int = 4, act: str = "bf16") -> int:
    """Tokens per block of the projection backward's dX / dW kernel (the partition of the token sum
    into per-block dW partials), chosen as the library chooses it."""
    K = n * C
    if n != 4:
        J = n * n + 2 * n
        by_budget = max(1, (512 << 20) // (K * J * 4))  # dW partials within 512 MiB
        if act == "f32":  # blocks of >= 64 tokens, at most 32 of them
            ntb = min(32, by_budget, max(1, _cdiv(N, 64)))
            return _cdiv(N, ntb)
        # bf16: about 512 workgroups over the tiles of the kernel that forms dW (64 or 128 channels of
        # all n streams for n <= 3, 256 consecutive k for n >= 5), blocks in whole 32-token sub-tiles
        tiles = _cdiv(K, 256) if n >= 5 else _cdiv(C, 32 * (4 if n <= 2 else 2))
        ntb = min(max(1, 512 // tiles), by_budget, max(1, _cdiv(N, 32)))
        return _rup(_cdiv(N, ntb), 32)
    if act == "f32":  # about 2048 workgroups of 1024 k
        return _rup(max(32, _cdiv(N * _cdiv(K, 1024), 2048)), 32)
    nkt = _cdiv(K, 256)  # bf16: whole rounds of 256 workgroups, then the fewest blocks
    best = (-1, 0, _rup(N, 32))
    for want in range(1, 65):
        tb = _rup(_cdiv(N, want), 32)
        nb = _cdiv(N, tb)
        fill = nb * nkt * 100 // _rup(nb * nkt, 256)
        if fill > best[0] or (fill == best[0] and nb < best[1]):
            best = (fill, nb, tb)
    return best[2]


def sum_depth(path: str, N: int, C: int = 0, S: int | None = None, n: int = 4, act: str = "bf16") -> int:
    """Longest chain of rounded fp32 operations that one token's nonzero contribution takes into a sum
    over tokens, for the reduction tree of the kernels on `path`.  S = the number of tokens whose
    contribution may be nonzero (N when None): adding an exact zero is exact, so a sequential walk
    rounds at most once per nonzero term it meets.  The leading 1 is the product forming the term.

      proj   dW, per token block of dxdw_token_block tokens, then the block partials summed in
             order.  bf16 (any n): at most six MFMA accumulations per 32 tokens (three bf16 terms of
             dp on each 16 tokens, one MFMA contracting 16 tokens) and at most 15 roundings
             inside one MFMA.  fp32: one fma (n = 4)
             or one add (other n) per token.
      param  dalpha, dhbias.  n = 4: <= 4 adds over a lane's owned columns, a 64-lane DPP tree (6),
             four waves (2), one thread's strided walk over 64-token block partials (every 32nd
             block), a 32-way tree (5).  Other n: a per-token row (<= n^2 adds in the RES segment),
             then 256 threads striding the rows, a 64-lane tree (6) and <= 8 waves in order.
      rows   fp32 dbias and dgamma: a workgroup's <= 64 tokens in order, then 16 slices of the
             partial rows in order, then the 16 slices in order.
      hpre   shared-row dH_pre: 256 threads striding the per-token rows, then a tree of depth 8
             (n = 4) or a 64-lane tree and <= 8 waves (other n).
    """
    idx = None
    if S is not None and np.ndim(S) == 1:  # the indices of the tokens with a nonzero contribution
        idx = np.unique(np.asarray(S, np.int64))
        S = len(idx)
    S = N if S is None else min(S, N)
    if path == "proj":
        tb = dxdw_token_block(N, C, n, act)
        nb = _cdiv(N, tb)
        bf = act == "bf16"
        if idx is not None:  # per block: its nonzero tokens (fp32) or 32-token sub-tiles (bf16 MFMA)
            blocks = idx // tb
            units = np.unique(idx // 32) // (tb // 32) if bf else blocks
            seq = int(np.bincount(units).max())
            return 1 + (15 + 6 * seq if bf else seq) + len(np.unique(blocks))
        if bf:
            return 1 + 15 + 6 * min(S, _cdiv(tb, 32)) + min(S, nb)
        return 1 + min(S, tb) + min(S, nb)
    if path == "param":
        if n == 4:
            return 1 + 4 + 6 + 2 + min(S, _cdiv(_cdiv(N, 64), 32)) + 5
        return 1 + n * n + min(S, _cdiv(N, 256)) + 6 + 8
    if path == "rows":
        R = _cdiv(N, 16)
        return 1 + min(S, 64) + min(S, _cdiv(R, 16) + 1) + min(S, 16)
    if path == "hpre":
        return 1 + min(S, _cdiv(N, 256)) + (8 if n == 4 else 14)
    raise ValueError(path)


def assert_tokensum(name, g, o, abs_parts, act="f32", depth=None):
    """Sum over tokens.  fp32: abs_parts = sum_t |o_t| (same shape as o) and depth = sum_depth(...) of
    the kernel path (see the module rules).  bf16: the bf16 rule alone (abs_parts unused)."""
    g = h64(g); o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (name, g.shape, o.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    rms = np.sqrt(np.mean(o * o)) if o.size else 0.0
    if act == "bf16":
        ob = O.round_f64_to_bf16(o)
        _report(name, g, ob, 8e-3 * np.abs(ob) + 1e-5 * rms)
    else:
        assert depth is not None, f"{name}: fp32 token sums need the reduction depth"
        s = np.asarray(abs_parts, np.float64)
        assert s.shape == o.shape, (name, s.shape, o.shape)
        _report(name, g, o, 1e-5 * (np.abs(o) + rms) + (1e-5 + gamma_fp32(depth)) * s)


def sinkhorn_rtol(iters: int, grad: bool, n: int = 4) -> float:
    """Relative tolerance of the Sinkhorn outputs (H_res: the rel rule; dlogits: the mixed rule).

    The stated 1e-5 holds for H_res at every iteration count tested (worst 0.28x of it at 200
    iterations, n = 4; 0.11x at 150 for the other n), and for the n = 4 gradient (0.57x at 200: its
    replay rebuilds at most 20 iterations from the logits).  The gradient of the other n gathers the
    rounding of its fp32 reverse pass linearly in the number of half-steps it walks: 0.5-0.6x of
    1e-5 at 45 iterations, 1.1-1.9x at 150 for n >= 3.  Beyond 50 iterations it is held to
    1e-5 iters / 50."""
    if not grad or n == 4 or iters <= 50:
        return 1e-5
    return 1e-5 * iters / 50


def h_res_chain_bound(L, iters, eps, tol_L):
    """First-order bound on |Sinkhorn(L') - Sinkhorn(L)| over all L' with |L' - L| <= tol_L elementwise:
    sum_cd |dH_ab / dL_cd| tol_L[cd], each Jacobian row taken from the oracle's reverse mode
    (one backward call per output entry).  L [N, n, n] (float64), tol_L broadcastable to it."""
    L = np.asarray(L, np.float64)
    N, n, _ = L.shape
    tol = np.broadcast_to(np.asarray(tol_L, np.float64), L.shape)
    b = np.empty_like(L)
    for a in range(n):
        for c in range(n):
            e = np.zeros_like(L)
            e[:, a, c] = 1.0
            b[:, a, c] = np.sum(np.abs(O.sinkhorn_bwd(e, L, iters, eps)) * tol, axis=(1, 2))
    return b


def assert_h_res(o_H_res, o_logits, ref_H_res, ref_L, iters, eps, alone=None):
    """The fused pre forward's H_res.  The oracle is never fed a GPU value:
      1. if `alone` (mhc_sinkhorn_fwd run on the same GPU logits) is given, bit for bit: the fused
         finalize's Sinkhorn (quad layout at n = 4, a matrix per lane elsewhere) is the same
         operation sequence as the standalone kernel, which the Sinkhorn tests hold to 1e-5 against
         the oracle on seeded logits;
      2. against the oracle's own H_res (from the seeded inputs), within 1e-5 relative plus the
         GPU's measured logit deviation from the oracle's logits carried through the Sinkhorn map to
         first order (sum_cd |dH_ab/dL_cd| |dL_cd|, the Jacobian from the oracle's reverse mode at the
         oracle's logits), with a 10% margin for the second-order terms."""
    if alone is not None:
        a, b = h64(o_H_res), h64(alone)
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64)), \
            "fused H_res differs from mhc_sinkhorn_fwd on the same logits"
    ref_L = np.asarray(ref_L, np.float64)
    dL = np.abs(h64(o_logits) - ref_L)
    g = h64(o_H_res); r = np.asarray(ref_H_res, np.float64)
    bound = 1e-5 * np.abs(r) + 1.1 * h_res_chain_bound(ref_L, iters, eps, dL)
    _report("H_res (against the oracle, logit deviation carried)", g, r, _fp32_floor(bound, r))


def norm_chain_bound(x, dx, gamma, eps):
    """First-order change of the RMSNorm output y = gamma x / (q + eps), q = sqrt(mean x^2), when its
    input row x [N, C] moves by dx: |gamma (r dx - x r^2 dq)| with dq = sum_c x dx / (C q) (0 for an
    all-zero row)."""
    x = np.asarray(x, np.float64); dx = np.asarray(dx, np.float64)
    C = x.shape[1]
    q = np.sqrt(np.mean(x * x, axis=1, keepdims=True))
    r = 1.0 / (q + eps)
    dq = np.where(q > 0, np.sum(x * dx, axis=1, keepdims=True) / (C * np.where(q > 0, q, 1.0)), 0.0)
    gm = 1.0 if gamma is None else np.asarray(gamma, np.float64)[None, :]
    return np.abs(gm * (r * dx - x * r * r * dq))


def assert_normed(name, g_normed, g_agg, ref_agg, gamma, eps, act):
    """The normalised output of the fused pre forward against the oracle's norm of its own stored
    (rounded) agg: one bf16 ulp (or the fp32 rule) plus the GPU's measured agg deviation from that
    stored agg carried through the norm to first order (norm_chain_bound, 10% margin).  The oracle is
    never fed a GPU value."""
    a_o = O.round_to(np.asarray(ref_agg, np.float64), act)
    yo, _ = O.rmsnorm_fwd(a_o, gamma, eps)
    carried = 1.1 * norm_chain_bound(a_o, h64(g_agg) - a_o, gamma, eps)
    g = h64(g_normed)
    rms = np.sqrt(np.mean(yo * yo)) if yo.size else 0.0
    if act == "bf16":
        ob = O.round_f64_to_bf16(yo)
        _report(name, g, ob, 8e-3 * np.abs(ob) + 1e-5 * rms + carried)
    else:
        _report(name, g, yo, _fp32_floor(1e-5 * (np.abs(yo) + rms) + carried, yo))


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
