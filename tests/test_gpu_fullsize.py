"""GPU parity at the full workload sizes, with the arguments bench.py passes.

The kernels run over every token, with the same grids as in the timed step;
the oracle checks a sample of tokens that it computes one by one:

  * per-token outputs (H tensors, logits, r/q/z, agg, out, dX, dH, dx) are
    compared on the sampled tokens;
  * for the sums over tokens (dW, dalpha, dhbias, dbias) the upstream
    gradients are nonzero only on the sampled tokens.  Every other token then
    contributes exact zeros (its gradients are exactly zero, checked on a
    second sample), so the oracle's sums over the sample are the expected
    values while the kernels still reduce over all token blocks.

The sample holds the first and last tokens, tokens on both sides of the
256- and 1024-token block edges, and random tokens.  Inputs are the seeded
synthetic workloads; derived inputs of an op under test (H_res, saved state)
come from the oracle, never from the GPU.
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (assert_act, assert_h_res, assert_mixed, assert_normed, assert_rel, assert_tokensum, dev,
                      h64, log, pre_bwd_abs_parts, sum_depth)
from mhc_hyper_connection_proj_amd import binding as B
from mhc_hyper_connection_proj_amd import synth

pytestmark = pytest.mark.gpu


def sample_tokens(N: int, seed: int, k: int = 24) -> np.ndarray:
    s = {0, 1, N - 2, N - 1}
    for edge in (256, 1024):
        for m in range(edge, N, edge * 5):
            s.update((m - 1, m))
    rng = np.random.default_rng(seed)
    s.update(int(t) for t in rng.choice(N, size=k, replace=False))
    return np.array(sorted(t for t in s if 0 <= t < N), dtype=np.int64)


def others(N: int, S: np.ndarray, seed: int, k: int = 16) -> np.ndarray:
    rng = np.random.default_rng(seed + 1)
    rest = np.setdiff1d(rng.choice(N, size=4 * k, replace=False), S)
    return np.sort(rest[:k])


def rows(t: torch.Tensor, idx: np.ndarray) -> torch.Tensor:
    return t[torch.from_numpy(idx).to(t.device)]


@functools.lru_cache(maxsize=3)
def residual(name: str) -> np.ndarray:
    w = synth.WORKLOADS[name]
    log(f"generating X for {name}: {w.tokens} x {w.n} x {w.C}")
    return synth.tensor(w, "X")


def only(a: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Copy of a with every token row outside S set to zero."""
    z = np.zeros_like(a)
    z[S] = a[S]
    return z


# ----------------------------------------------------------------- pre pass forward
@pytest.mark.parametrize("name", ["full_layer", "pre_fwd"])
def test_pre_fwd_full_size(name):
    w = synth.WORKLOADS[name]
    N = w.tokens
    log(f"pre fwd full size {name}: N={N} C={w.C}")
    X = residual(name)
    W = synth.tensor(w, "W")
    o = B.mhc_pre_fwd(dev(X), dev(W), None, None, w.rms_eps, w.iters, w.eps)
    torch.cuda.synchronize()
    S = sample_tokens(N, w.wid)
    ref = O.pre_fwd(h64(X[S]), h64(W), None, None, w.rms_eps, w.iters, w.eps)
    assert_rel("H_pre", rows(o["H_pre"], S), ref["H_pre"])
    assert_rel("H_post", rows(o["H_post"], S), ref["H_post"])
    assert_mixed("logits", rows(o["H_res_logits"], S), ref["L"])
    assert_h_res(rows(o["H_res"], S), rows(o["H_res_logits"], S), ref["H_res"], ref["L"], w.iters, w.eps,
                 alone=B.mhc_sinkhorn_fwd(rows(o["H_res_logits"], S).contiguous(), w.iters, w.eps))
    sv = h64(rows(o["saved"], S))
    assert_rel("r", sv[:, 0], ref["r"])
    assert_rel("q", sv[:, 1], ref["q"])
    assert_mixed("z", sv[:, 2:26], ref["z"])
    assert_act("agg", rows(o["agg"], S), ref["agg"], w.act)
    # the VALU (FMA) form of the projection at the same size
    Hp, Hq, L, sv2 = B.mhc_proj_rms_h_fma(dev(X), dev(W), None, None, w.rms_eps)
    torch.cuda.synchronize()
    assert_rel("H_pre (fma)", rows(Hp, S), ref["H_pre"])
    assert_rel("H_post (fma)", rows(Hq, S), ref["H_post"])
    assert_mixed("logits (fma)", rows(L, S), ref["L"])
    assert_rel("r (fma)", h64(rows(sv2, S))[:, 0], ref["r"])


# ----------------------------------------------------------------- post (h_post_bda) forward + backward
@pytest.mark.parametrize("name", ["full_layer", "post_bda"])
def test_post_bda_full_size(name):
    w = synth.WORKLOADS[name]
    N, C = w.tokens, w.C
    log(f"post fwd/bwd full size {name}: N={N} C={C} bias={w.has_bias}")
    X = residual(name)
    x = synth.tensor(w, "x")
    bias = synth.tensor(w, "bias") if w.has_bias else None
    H_res = O.round_f64_to_f32(O.sinkhorn_fwd(h64(synth.tensor(w, "L")), w.iters, w.eps)).astype(np.float32)
    lg = synth.tensor(w, "Hpost_logits").astype(np.float64)
    H_post = (2.0 / (1.0 + np.exp(-lg))).astype(np.float32)  # input synthesis: a positive gate in (0, 2)
    S = sample_tokens(N, w.wid)
    Z = others(N, S, w.wid)
    G = only(synth.tensor(w, "G"), S)
    Xd, Hr, Hp, xd = dev(X), dev(H_res), dev(H_post), dev(x)
    bd = dev(bias) if bias is not None else None
    out = B.mhc_h_post_bda_fwd(Xd, Hr, Hp, xd, bd)
    dX, dHr, dHp, dx, db = B.mhc_h_post_bda_bwd(dev(G), Xd, Hr, Hp, xd, bd)
    torch.cuda.synchronize()
    bias64 = h64(bias) if bias is not None else None
    ro = O.h_post_bda_fwd(h64(X[S]), h64(H_res[S]), h64(H_post[S]), h64(x[S]), bias64)
    rdX, rdHr, rdHp, rdx, rdb = O.h_post_bda_bwd(h64(G[S]), h64(X[S]), h64(H_res[S]), h64(H_post[S]),
                                                 h64(x[S]), bias64)
    assert_act("out", rows(out, S), ro, w.act)
    assert_act("dX", rows(dX, S), rdX, w.act)
    assert_mixed("dH_res", rows(dHr, S), rdHr)
    assert_mixed("dH_post", rows(dHp, S), rdHp)
    assert_act("dx", rows(dx, S), rdx, w.act)
    for nm, t in (("dX", dX), ("dH_res", dHr), ("dH_post", dHp), ("dx", dx)):
        assert not h64(rows(t, Z)).any(), f"{nm}: nonzero on tokens with zero upstream gradient"
    if bias is not None:
        assert_tokensum("dbias", db, rdb, np.abs(rdx).sum(axis=0), w.act, sum_depth("rows", N, S=len(S)))
    # as timed: no dX (the pre backward forms it) and no dbias
    _, dHr2, dHp2, dx2, _ = B.mhc_h_post_bda_bwd(dev(G), Xd, Hr, Hp, xd, bd, want_dbias=False, want_dX=False)
    torch.cuda.synchronize()
    assert_mixed("dH_res (no dX)", rows(dHr2, S), rdHr)
    assert_mixed("dH_post (no dX)", rows(dHp2, S), rdHp)
    assert_act("dx (no dX)", rows(dx2, S), rdx, w.act)
    for nm, t in (("dH_res", dHr2), ("dH_post", dHp2), ("dx", dx2)):
        assert not h64(rows(t, Z)).any(), f"{nm} (no dX): nonzero on tokens with zero upstream gradient"


# ----------------------------------------------------------------- pre pass backward
@pytest.mark.parametrize("name,mode", [("full_layer", "post"), ("full_layer", "accumulate"), ("pre_fwd", "post")])
def test_pre_bwd_full_size(name, mode):
    w = synth.WORKLOADS[name]
    N, C, n = w.tokens, w.C, w.n
    log(f"pre bwd full size {name}: N={N} C={C} mode={mode}")
    X = residual(name)
    W = synth.tensor(w, "W")
    S = sample_tokens(N, w.wid)
    Z = others(N, S, w.wid)
    ref = O.pre_fwd(h64(X[S]), h64(W), None, None, w.rms_eps, w.iters, w.eps)
    # forward state: the oracle's on the sampled tokens; any finite values
    # elsewhere (their upstream gradients are zero)
    saved = np.zeros((N, 32), np.float32); saved[:, 0] = 1.0; saved[:, 1] = 1.0
    saved[S, 0] = ref["r"]; saved[S, 1] = ref["q"]; saved[S, 2:26] = ref["z"]
    H_pre = np.full((N, n), 0.25, np.float32); H_pre[S] = ref["H_pre"]
    H_post = np.ones((N, n), np.float32); H_post[S] = ref["H_post"]
    L = np.zeros((N, n, n), np.float32); L[S] = ref["L"]
    rng = np.random.default_rng(w.wid + 50)
    g = only(synth.tensor(w, "x"), S)
    dHp = np.zeros((N, n), np.float32); dHp[S] = rng.standard_normal((len(S), n))
    dHr = np.zeros((N, n, n), np.float32); dHr[S] = rng.standard_normal((len(S), n, n))
    if mode == "accumulate":  # the post pass's dX, materialised and accumulated onto
        dX0 = synth.tensor(w, "G")
        ob = B.mhc_pre_bwd(dev(g), dev(dHp), dev(dHr), dev(X), dev(W), dev(saved), dev(H_pre), dev(H_post),
                           dev(L), alpha=None, iters=w.iters, eps=w.eps, dX=dev(dX0), accumulate_dX=True)
        base_S, base_Z = h64(dX0[S]), h64(dX0[Z])
    else:  # as timed: the post pass's dX term formed here from its G (all tokens) and H_res
        Gp = synth.tensor(w, "G")
        Hrp = O.round_f64_to_f32(O.sinkhorn_fwd(h64(synth.tensor(w, "L")), w.iters, w.eps)).astype(np.float32)
        ob = B.mhc_pre_bwd(dev(g), dev(dHp), dev(dHr), dev(X), dev(W), dev(saved), dev(H_pre), dev(H_post),
                           dev(L), alpha=None, iters=w.iters, eps=w.eps, post_G=dev(Gp), post_H_res=dev(Hrp))
        zero4, zc = np.zeros((len(S), n)), np.zeros((len(S), C))
        base_S = O.h_post_bda_bwd(h64(Gp[S]), h64(X[S]), h64(Hrp[S]), zero4, zc)[0]
        zero4, zc = np.zeros((len(Z), n)), np.zeros((len(Z), C))
        base_Z = O.round_f64_to_bf16(O.h_post_bda_bwd(h64(Gp[Z]), h64(X[Z]), h64(Hrp[Z]), zero4, zc)[0])
    torch.cuda.synchronize()
    rb = O.pre_bwd(h64(g[S]), h64(dHp[S]), h64(dHr[S]), h64(X[S]), h64(W), None, None, w.rms_eps, w.iters, w.eps)
    assert_act("dX", rows(ob["dX"], S), base_S + rb["dX"], w.act)
    if mode == "accumulate":
        assert np.array_equal(h64(rows(ob["dX"], Z)), base_Z), "dX changed on tokens with zero gradient"
    else:  # zero pre-pass gradient there: dX is the post term alone
        assert_act("dX (post term only)", rows(ob["dX"], Z), base_Z, w.act)
    aW, aa, ab = pre_bwd_abs_parts(h64(g[S]), h64(dHp[S]), h64(dHr[S]), h64(X[S]), h64(W), None, None, w.rms_eps,
                                   w.iters, w.eps)
    assert_tokensum("dW", ob["dW"], rb["dW"], aW, depth=sum_depth("proj", N, C, S=S))
    assert_tokensum("dalpha", ob["dalpha"], rb["dalpha"], aa, depth=sum_depth("param", N, S=len(S)))
    assert_tokensum("dhbias", ob["dhbias"], rb["dhbias"], ab, depth=sum_depth("param", N, S=len(S)))


# ----------------------------------------------------------------- stream mix / distribute, shared-row aggregate
def test_variants_full_size():
    w = synth.WORKLOADS["full_layer"]
    N, C, n = w.tokens, w.C, w.n
    log(f"variants full size: N={N} C={C}")
    X = residual("full_layer")
    S = sample_tokens(N, w.wid + 7)
    Z = others(N, S, w.wid + 7)
    rng = np.random.default_rng(w.wid + 70)
    G = only(synth.tensor(w, "G"), S)
    x = synth.tensor(w, "x")
    M = rng.standard_normal((N, n, n)).astype(np.float32)
    Hp = rng.standard_normal((N, n)).astype(np.float32)
    h = np.array([0.4, -0.3, 0.2, 0.7], np.float32)
    Xd, Gd, xd = dev(X), dev(G), dev(x)
    out_m = B.mhc_stream_mix_fwd(Xd, dev(M))
    dX_m, dM_m = B.mhc_stream_mix_bwd(Gd, Xd, dev(M))
    out_d = B.mhc_stream_distribute_fwd(xd, dev(Hp))
    dx_d, dH_d = B.mhc_stream_distribute_bwd(Gd, xd, dev(Hp))
    agg_s = B.mhc_h_aggregate_static_fwd(Xd, dev(h))
    g = only(x, S)  # upstream gradient on the sampled tokens only
    dX_s, dH_s = B.mhc_h_aggregate_static_bwd(dev(g), Xd, dev(h))
    torch.cuda.synchronize()
    XS, GS, xS = h64(X[S]), h64(G[S]), h64(x[S])
    assert_act("mix out", rows(out_m, S), O.stream_mix_fwd(XS, h64(M[S])), w.act)
    odX, odM = O.stream_mix_bwd(GS, XS, h64(M[S]))
    assert_act("mix dX", rows(dX_m, S), odX, w.act)
    assert_mixed("mix dM", rows(dM_m, S), odM)
    assert_act("dist out", rows(out_d, S), O.stream_distribute_fwd(xS, h64(Hp[S])), w.act)
    odx, odH = O.stream_distribute_bwd(GS, xS, h64(Hp[S]))
    assert_act("dist dx", rows(dx_d, S), odx, w.act)
    assert_mixed("dist dH_post", rows(dH_d, S), odH)
    for nm, t in (("mix dX", dX_m), ("mix dM", dM_m), ("dist dx", dx_d), ("dist dH_post", dH_d)):
        assert not h64(rows(t, Z)).any(), f"{nm}: nonzero on tokens with zero upstream gradient"
    assert_act("static agg", rows(agg_s, S), O.h_aggregate_static_fwd(XS, h64(h)), w.act)
    sdX, sdH = O.h_aggregate_static_bwd(h64(g[S]), XS, h64(h))
    assert_act("static dX", rows(dX_s, S), sdX, w.act)
    parts = np.abs(O.h_aggregate_bwd(h64(g[S]), XS, np.broadcast_to(h64(h), (len(S), n)).copy())[1]).sum(axis=0)
    assert_tokensum("static dH_pre", dH_s, sdH, parts, depth=sum_depth("hpre", N, S=len(S)))


# ----------------------------------------------------------------- RMSNorm of the aggregated stream
def test_rmsnorm_full_size():
    """Standalone norm fwd/bwd at 16384 x 7168 (bf16) and the fused pre pass + norm at full size."""
    w = synth.WORKLOADS["full_layer"]
    N, C = w.tokens, w.C
    log(f"rmsnorm full size: N={N} C={C}")
    S = sample_tokens(N, w.wid + 9)
    Z = others(N, S, w.wid + 9)
    x = synth.tensor(w, "x")
    gamma = synth.tensor(w, "gamma")
    dy = only(synth.tensor(w, "dy"), S)
    xd, gd = dev(x), dev(gamma)
    y = B.mhc_rmsnorm_fwd(xd, gd, w.rms_eps)
    dx, dg = B.mhc_rmsnorm_bwd(dev(dy), xd, gd, w.rms_eps)
    torch.cuda.synchronize()
    xS = h64(x[S])
    yo, r = O.rmsnorm_fwd(xS, h64(gamma), w.rms_eps)
    assert_act("y", rows(y, S), yo, w.act)
    dxo, dgo = O.rmsnorm_bwd(h64(dy[S]), xS, h64(gamma), w.rms_eps)
    assert_act("dx", rows(dx, S), dxo, w.act)
    assert not h64(rows(dx, Z)).any(), "dx: nonzero on tokens with zero upstream gradient"
    assert_tokensum("dgamma", dg, dgo, np.abs(h64(dy[S]) * r[:, None] * xS).sum(0), depth=sum_depth("rows", N, S=len(S)))
    del y, dx, dg, xd

    X = residual("full_layer")
    W = synth.tensor(w, "W")
    f = B.mhc_pre_rmsnorm_fwd(dev(X), dev(W), gd, None, None, w.rms_eps, w.iters, w.eps, w.rms_eps)
    torch.cuda.synchronize()
    ref = O.pre_fwd(h64(X[S]), h64(W), None, None, w.rms_eps, w.iters, w.eps)
    assert_act("agg", rows(f["agg"], S), ref["agg"], w.act)
    assert_rel("H_res", rows(f["H_res"], S), ref["H_res"])
    assert_normed("normed", rows(f["normed"], S), rows(f["agg"], S), ref["agg"], h64(gamma), w.rms_eps, w.act)


# ----------------------------------------------------------------- general n at the bench's shapes
@functools.lru_cache(maxsize=1)
def _gn_inputs(n: int, C: int, N: int = 16384):
    """Seeded N(0,1) bf16 residual and upstream gradient, W ~ N(0, 0.02^2): the shapes the bench's general-n
    step runs (no workload of the pages has n != 4)."""
    rng = np.random.Generator(np.random.PCG64(9000 + n))
    X = synth.f32_to_bf16_bits(rng.standard_normal((N, n, C), dtype=np.float32))
    G = synth.f32_to_bf16_bits(rng.standard_normal((N, n, C), dtype=np.float32))
    W = (rng.standard_normal((n * C, n * n + 2 * n), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((N, C), dtype=np.float32))
    return X, G, W, x


@pytest.mark.parametrize("n,C", [(2, 7168), (8, 2048)])
def test_general_n_full_size(n, C):
    """The whole step at 16384 tokens, as the bench times it for n != 4, on sampled tokens: pre forward,
    h_post_bda forward and backward (oracle H_res / H_post), pre backward with the h_post_bda term
    (oracle forward state on the sample, zero upstream gradients elsewhere)."""
    N, J, iters, eps = 16384, n * n + 2 * n, 20, 1e-6
    log(f"general n full size: n={n} N={N} C={C}")
    X, G, W, x = _gn_inputs(n, C)
    S = sample_tokens(N, 100 + n)
    Z = others(N, S, 100 + n)
    Xd = dev(X)
    o = B.mhc_pre_fwd(Xd, dev(W), None, None, 1e-6, iters, eps)
    torch.cuda.synchronize()
    ref = O.pre_fwd(h64(X[S]), h64(W), None, None, 1e-6, iters, eps)
    assert_rel("H_pre", rows(o["H_pre"], S), ref["H_pre"])
    assert_rel("H_post", rows(o["H_post"], S), ref["H_post"])
    assert_mixed("logits", rows(o["H_res_logits"], S), ref["L"])
    assert_h_res(rows(o["H_res"], S), rows(o["H_res_logits"], S), ref["H_res"], ref["L"], iters, eps,
                 alone=B.mhc_sinkhorn_fwd(rows(o["H_res_logits"], S).contiguous(), iters, eps))
    sv = h64(rows(o["saved"], S))
    assert_rel("r", sv[:, 0], ref["r"])
    assert_mixed("z", sv[:, 2:2 + J], ref["z"])
    assert_act("agg", rows(o["agg"], S), ref["agg"], "bf16")
    del o
    # h_post_bda on the oracle's H_res / H_post of the sample (finite stand-ins elsewhere)
    Hr = np.broadcast_to(np.eye(n, dtype=np.float32) * 0.5 + 0.5 / n, (N, n, n)).copy()
    Hp = np.ones((N, n), np.float32)
    Hr[S] = O.round_f64_to_f32(ref["H_res"]); Hp[S] = O.round_f64_to_f32(ref["H_post"])
    Gs = only(G, S)
    out = B.mhc_h_post_bda_fwd(Xd, dev(Hr), dev(Hp), dev(x))
    _, dHr, dHp, dx, _ = B.mhc_h_post_bda_bwd(dev(Gs), Xd, dev(Hr), dev(Hp), dev(x), None, want_dX=False)
    torch.cuda.synchronize()
    XS, GS, xS = h64(X[S]), h64(Gs[S]), h64(x[S])
    assert_act("out", rows(out, S), O.h_post_bda_fwd(XS, h64(Hr[S]), h64(Hp[S]), xS), "bf16")
    _, odHr, odHp, odx, _ = O.h_post_bda_bwd(GS, XS, h64(Hr[S]), h64(Hp[S]), xS)
    assert_mixed("dH_res", rows(dHr, S), odHr)
    assert_mixed("dH_post", rows(dHp, S), odHp)
    assert_act("dx", rows(dx, S), odx, "bf16")
    for nm, t in (("dH_res", dHr), ("dH_post", dHp), ("dx", dx)):
        assert not h64(rows(t, Z)).any(), f"{nm}: nonzero on tokens with zero upstream gradient"
    del out
    # the pre backward as the bench runs it: the h_post_bda term formed from G (all tokens)
    saved = np.zeros((N, B.saved_stride(n)), np.float32); saved[:, 0] = 1.0; saved[:, 1] = 1.0
    saved[S, 0] = ref["r"]; saved[S, 1] = ref["q"]; saved[S, 2:2 + J] = ref["z"]
    H_pre = np.full((N, n), 1.0 / n, np.float32); H_pre[S] = ref["H_pre"]
    H_post = np.ones((N, n), np.float32); H_post[S] = ref["H_post"]
    L = np.zeros((N, n, n), np.float32); L[S] = ref["L"]
    rng = np.random.default_rng(200 + n)
    g = only(x, S)
    dHq = np.zeros((N, n), np.float32); dHq[S] = rng.standard_normal((len(S), n))
    dHR = np.zeros((N, n, n), np.float32); dHR[S] = rng.standard_normal((len(S), n, n))
    ob = B.mhc_pre_bwd(dev(g), dev(dHq), dev(dHR), Xd, dev(W), dev(saved), dev(H_pre), dev(H_post), dev(L),
                       iters=iters, eps=eps, post_G=dev(G), post_H_res=dev(Hr))
    torch.cuda.synchronize()
    rb = O.pre_bwd(h64(g[S]), h64(dHq[S]), h64(dHR[S]), XS, h64(W), None, None, 1e-6, iters, eps)
    base_S = O.stream_mix_bwd(h64(G[S]), XS, h64(Hr[S]))[0]
    assert_act("dX", rows(ob["dX"], S), base_S + rb["dX"], "bf16")
    base_Z = O.stream_mix_bwd(h64(G[Z]), h64(X[Z]), h64(Hr[Z]))[0]
    assert_act("dX (post term only)", rows(ob["dX"], Z), base_Z, "bf16")
    aW, aa, ab = pre_bwd_abs_parts(h64(g[S]), h64(dHq[S]), h64(dHR[S]), XS, h64(W), None, None, 1e-6, iters, eps)
    assert_tokensum("dW", ob["dW"], rb["dW"], aW, depth=sum_depth("proj", N, C, S=S, n=n))
    assert_tokensum("dalpha", ob["dalpha"], rb["dalpha"], aa, depth=sum_depth("param", N, S=len(S), n=n))
    assert_tokensum("dhbias", ob["dhbias"], rb["dhbias"], ab, depth=sum_depth("param", N, S=len(S), n=n))
