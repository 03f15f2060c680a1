"""GPU parity for stream counts other than 4 (1 <= n <= 8), every entry point
against the fp64 oracle, which takes any n.  n = 4 (every benchmark workload)
runs on the kernels laid out for it and is covered by the other test files;
these cases exercise the kernels templated on n, with 1, 2 and 3 column
tiles of the projection (J = 3, 8, 15, 35, 80) and ragged token/channel counts.
Inputs are seeded synthetic arrays or oracle outputs; nothing fed to the oracle
comes from the GPU.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (assert_act, assert_h_res, assert_mixed, assert_rel, assert_tokensum, dev, h64, log,
                      sinkhorn_rtol, sum_depth)
from mhc_hyper_connection_proj_amd import binding as B

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(23)
NS = [1, 2, 3, 5, 6, 7, 8]


def f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def store(a64, act):
    return O.round_f64_to_bf16_bits(a64) if act == "bf16" else f32(a64)


def sig(v):
    return 1 / (1 + np.exp(-v))


@pytest.mark.parametrize("n", NS)
@pytest.mark.parametrize("iters,eps,std", [(20, 1e-6, 1.0), (0, 1e-6, 1.0), (1, 1e-6, 2.0), (7, 0.25, 1.0),
                                           (45, 1e-6, 1.0), (150, 0.25, 1.0)])
def test_sinkhorn_general_n(n, iters, eps, std):
    # The backward keeps every half-step's line sums in LDS: for n >= 3 with a row per lane where its
    # records fit (20 and 45 iterations here), else (and for n <= 2) with one token per lane where they
    # fit, else it replays the forward from checkpoints (150 iterations at n >= 3): all three paths run.
    # The fp32 reverse pass gathers rounding over the half-steps it walks: beyond 50 iterations the
    # gradient's bound grows with the iteration count (sinkhorn_rtol); H_res holds 1e-5 throughout.
    log(f"sinkhorn n={n} iters={iters} eps={eps}")
    count = 301
    L = f32(RNG.standard_normal((count, n, n)) * std)
    dH = f32(RNG.standard_normal((count, n, n)))
    H = B.mhc_sinkhorn_fwd(dev(L), iters, eps)
    dL = B.mhc_sinkhorn_bwd(dev(dH), dev(L), iters, eps)
    torch.cuda.synchronize()
    oH, odL = O.sinkhorn_fwd(h64(L), iters, eps), O.sinkhorn_bwd(h64(dH), h64(L), iters, eps)
    rms = np.sqrt(np.mean(odL * odL))
    log(f"  worst error / 1e-5 bound: H_res {np.max(np.abs(h64(H) - oH) / np.maximum(1e-5 * np.abs(oH), 1e-300)):.3f}, "
        f"dlogits {np.max(np.abs(h64(dL) - odL) / np.maximum(1e-5 * (np.abs(odL) + rms), 1e-300)):.3f}")
    assert_rel("H_res", H, oH)
    assert_mixed("dlogits", dL, odL, rtol=sinkhorn_rtol(iters, grad=True, n=n))


@pytest.mark.parametrize("n", NS)
@pytest.mark.parametrize("act,N,C", [("bf16", 37, 296), ("f32", 9, 1032), ("bf16", 3, 8), ("bf16", 5, 4096)])
def test_streaming_ops_general_n(n, act, N, C):
    log(f"streaming n={n} act={act} N={N} C={C}")
    X = store(RNG.standard_normal((N, n, C)), act)
    G = store(RNG.standard_normal((N, n, C)), act)
    x = store(RNG.standard_normal((N, C)), act)
    g = store(RNG.standard_normal((N, C)), act)
    b = store(RNG.standard_normal(C) * 0.1, act)
    dX0 = store(RNG.standard_normal((N, n, C)), act)
    Hpre = f32(sig(RNG.standard_normal((N, n))))
    Hr = f32(O.sinkhorn_fwd(RNG.standard_normal((N, n, n)), 20, 1e-6))
    Hp = f32(2 * sig(RNG.standard_normal((N, n))))
    h = f32(RNG.uniform(-1, 1, n))
    Xd, Gd, xd = dev(X), dev(G), dev(x)
    agg = B.mhc_h_aggregate_fwd(Xd, dev(Hpre))
    adX, adH = B.mhc_h_aggregate_bwd(dev(g), Xd, dev(Hpre))
    adXa, _ = B.mhc_h_aggregate_bwd(dev(g), Xd, dev(Hpre), dX=dev(dX0), accumulate_dX=True)
    out = B.mhc_h_post_bda_fwd(Xd, dev(Hr), dev(Hp), xd, dev(b))
    pdX, pdHr, pdHp, pdx, pdb = B.mhc_h_post_bda_bwd(Gd, Xd, dev(Hr), dev(Hp), xd, dev(b))
    _, qdHr, qdHp, qdx, _ = B.mhc_h_post_bda_bwd(Gd, Xd, dev(Hr), dev(Hp), xd, None, want_dX=False)
    mo = B.mhc_stream_mix_fwd(Xd, dev(Hr))
    mdX, mdM = B.mhc_stream_mix_bwd(Gd, Xd, dev(Hr))
    do = B.mhc_stream_distribute_fwd(xd, dev(Hp))
    ddx, ddH = B.mhc_stream_distribute_bwd(Gd, xd, dev(Hp))
    so = B.mhc_h_aggregate_static_fwd(Xd, dev(h))
    sdX, sdH = B.mhc_h_aggregate_static_bwd(dev(g), Xd, dev(h))
    torch.cuda.synchronize()
    X64, G64, x64, g64, b64 = h64(X), h64(G), h64(x), h64(g), h64(b)
    assert_act("agg", agg, O.h_aggregate_fwd(X64, h64(Hpre)), act)
    odX, odH = O.h_aggregate_bwd(g64, X64, h64(Hpre))
    assert_act("agg dX", adX, odX, act)
    assert_act("agg dX accumulated", adXa, h64(dX0) + odX, act)
    assert_mixed("dH_pre", adH, odH)
    assert_act("post out", out, O.h_post_bda_fwd(X64, h64(Hr), h64(Hp), x64, b64), act)
    o = O.h_post_bda_bwd(G64, X64, h64(Hr), h64(Hp), x64, b64)
    assert_act("post dX", pdX, o[0], act)
    assert_mixed("post dH_res", pdHr, o[1])
    assert_mixed("post dH_post", pdHp, o[2])
    assert_act("post dx", pdx, o[3], act)
    assert_tokensum("post dbias", pdb, o[4], np.abs(o[3]).sum(axis=0), act, sum_depth("rows", N))
    o2 = O.h_post_bda_bwd(G64, X64, h64(Hr), h64(Hp), x64, None)
    assert_mixed("post dH_res (no dX, no bias)", qdHr, o2[1])
    assert_mixed("post dH_post (no dX, no bias)", qdHp, o2[2])
    assert_act("post dx (no dX, no bias)", qdx, o2[3], act)
    assert_act("mix out", mo, O.stream_mix_fwd(X64, h64(Hr)), act)
    omX, omM = O.stream_mix_bwd(G64, X64, h64(Hr))
    assert_act("mix dX", mdX, omX, act)
    assert_mixed("mix dM", mdM, omM)
    assert_act("dist out", do, O.stream_distribute_fwd(x64, h64(Hp)), act)
    odx, odH2 = O.stream_distribute_bwd(G64, x64, h64(Hp))
    assert_act("dist dx", ddx, odx, act)
    assert_mixed("dist dH_post", ddH, odH2)
    assert_act("static agg", so, O.h_aggregate_static_fwd(X64, h64(h)), act)
    osX, osH = O.h_aggregate_static_bwd(g64, X64, h64(h))
    assert_act("static dX", sdX, osX, act)
    parts = np.abs(O.h_aggregate_bwd(g64, X64, np.broadcast_to(h64(h), (N, n)).copy())[1]).sum(axis=0)
    assert_tokensum("static dH_pre", sdH, osH, parts, depth=sum_depth("hpre", N, n=n))


def _proj_inputs(n, act, N, C, zero_row=False):
    X = store(RNG.standard_normal((N, n, C)), act)
    if zero_row and N > 3:
        X[2] = 0
    J = n * n + 2 * n
    W = f32(RNG.standard_normal((n * C, J)) * 0.02)
    alpha = f32([1.3, 0.7, 1.1])
    hb = f32(RNG.standard_normal(J) * 0.1)
    return X, W, alpha, hb


def _abs_parts_pre(g, dHq, dHr, X, W, alpha, hb):
    aW = aa = ab = 0.0
    for t in range(X.shape[0]):
        r = O.pre_bwd(g[t:t + 1], dHq[t:t + 1], dHr[t:t + 1], X[t:t + 1], W, alpha, hb, 1e-6, 20, 1e-6)
        aW = aW + np.abs(r["dW"]); aa = aa + np.abs(r["dalpha"]); ab = ab + np.abs(r["dhbias"])
    return aW, aa, ab


@pytest.mark.parametrize("n", NS)
@pytest.mark.parametrize("act,N,C", [("f32", 40, 256), ("bf16", 37, 296), ("bf16", 70, 1032), ("bf16", 9, 16)])
def test_proj_rms_h_general_n(n, act, N, C):
    log(f"proj n={n} act={act} N={N} C={C}")
    X, W, alpha, hb = _proj_inputs(n, act, N, C, zero_row=True)
    J = n * n + 2 * n
    Hp, Hq, L, saved = B.mhc_proj_rms_h(dev(X), dev(W), dev(alpha), dev(hb), 1e-6)
    torch.cuda.synchronize()
    p = O.proj_rms_h(h64(X), h64(W), h64(alpha), h64(hb), 1e-6)
    s = h64(saved)
    assert s.shape[1] == B.saved_stride(n)
    assert_rel("q", s[:, 1], p.q)
    assert_rel("r", s[:, 0], p.r)
    assert_mixed("z", s[:, 2:2 + J], p.z)
    np.testing.assert_array_equal(s[:, 2 + J:], 0.0)
    assert_mixed("logits", L, p.L)
    assert_rel("H_pre", Hp, p.H_pre)
    assert_rel("H_post", Hq, p.H_post)
    # backward from the oracle's saved state
    sv = np.zeros((N, B.saved_stride(n)), np.float32)
    sv[:, 0] = p.r; sv[:, 1] = p.q; sv[:, 2:2 + J] = p.z
    dHp = f32(RNG.standard_normal((N, n))); dHq = f32(RNG.standard_normal((N, n)))
    dL = f32(RNG.standard_normal((N, n, n)))
    dX0 = store(RNG.standard_normal((N, n, C)), act)
    args = (dev(X), dev(W), dev(sv), dev(f32(p.H_pre)), dev(f32(p.H_post)), dev(dHp), dev(dHq), dev(dL))
    dX, dW, da, db = B.mhc_proj_rms_h_bwd(*args, alpha=dev(alpha))
    dXa, _, _, _ = B.mhc_proj_rms_h_bwd(*args, alpha=dev(alpha), dX=dev(dX0), accumulate_dX=True,
                                        want_dW=False, want_dalpha=False, want_dhbias=False)
    torch.cuda.synchronize()
    odX, odW, oda, odb = O.proj_rms_h_bwd(h64(X), h64(W), h64(dHp), h64(dHq), h64(dL), h64(alpha), h64(hb), 1e-6)
    assert_act("dX", dX, odX, act)
    assert_act("dX accumulated", dXa, h64(dX0) + odX, act)
    aW = aa = ab = 0.0
    for t in range(N):
        _, w_, a_, b_ = O.proj_rms_h_bwd(h64(X)[t:t + 1], h64(W), h64(dHp)[t:t + 1], h64(dHq)[t:t + 1],
                                         h64(dL)[t:t + 1], h64(alpha), h64(hb), 1e-6)
        aW = aW + np.abs(w_); aa = aa + np.abs(a_); ab = ab + np.abs(b_)
    assert_tokensum("dW", dW, odW, aW, depth=sum_depth("proj", N, C, n=n, act=act))
    assert_tokensum("dalpha", da, oda, aa, depth=sum_depth("param", N, n=n))
    assert_tokensum("dhbias", db, odb, ab, depth=sum_depth("param", N, n=n))


@pytest.mark.parametrize("n,C", [(1, 16384), (2, 8192), (3, 8192)])
def test_proj_staggered_walk_general_n(n, C):
    """Rows a multiple of 16 KB apart (and at least 32 KB) take the staggered projection walk; 1030
    tokens make five token blocks, so the walk starts at every one of its four sub-slices."""
    N, act = 1030, "bf16"
    log(f"proj staggered n={n} N={N} C={C}")
    X, W, alpha, hb = _proj_inputs(n, act, N, C, zero_row=True)
    J = n * n + 2 * n
    Hp, Hq, L, saved = B.mhc_proj_rms_h(dev(X), dev(W), dev(alpha), dev(hb), 1e-6)
    torch.cuda.synchronize()
    p = O.proj_rms_h(h64(X), h64(W), h64(alpha), h64(hb), 1e-6)
    s = h64(saved)
    assert_rel("q", s[:, 1], p.q)
    assert_rel("r", s[:, 0], p.r)
    assert_mixed("z", s[:, 2:2 + J], p.z)
    assert_mixed("logits", L, p.L)
    assert_rel("H_pre", Hp, p.H_pre)
    assert_rel("H_post", Hq, p.H_post)


@pytest.mark.parametrize("n", NS)
@pytest.mark.parametrize("mode", ["accumulate", "post"])
@pytest.mark.parametrize("act,N,C", [("bf16", 37, 296), ("f32", 20, 256), ("bf16", 66, 2048)])
def test_pre_fwd_bwd_general_n(n, act, N, C, mode):
    log(f"pre n={n} act={act} N={N} C={C} mode={mode}")
    X, W, alpha, hb = _proj_inputs(n, act, N, C)
    J = n * n + 2 * n
    o = B.mhc_pre_fwd(dev(X), dev(W), dev(alpha), dev(hb), 1e-6, 20, 1e-6)
    on = B.mhc_pre_rmsnorm_fwd(dev(X), dev(W), None, dev(alpha), dev(hb), 1e-6, 20, 1e-6, 1e-6)
    torch.cuda.synchronize()
    ref = O.pre_fwd(h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    assert_rel("H_pre", o["H_pre"], ref["H_pre"])
    assert_rel("H_post", o["H_post"], ref["H_post"])
    assert_mixed("logits", o["H_res_logits"], ref["L"])
    assert_h_res(o["H_res"], o["H_res_logits"], ref["H_res"], ref["L"], 20, 1e-6,
                 alone=B.mhc_sinkhorn_fwd(o["H_res_logits"], 20, 1e-6))
    assert_act("agg", o["agg"], ref["agg"], act)
    for k in ("H_pre", "H_post", "H_res", "agg"):
        assert torch.equal(o[k], on[k]), k
    alone = B.mhc_rmsnorm_fwd(o["agg"], None, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(on["normed"], alone)
    sv = np.zeros((N, B.saved_stride(n)), np.float32)
    sv[:, 0] = ref["r"]; sv[:, 1] = ref["q"]; sv[:, 2:2 + J] = ref["z"]
    g = store(RNG.standard_normal((N, C)), act)
    dHq = f32(RNG.standard_normal((N, n)))
    dHr = f32(RNG.standard_normal((N, n, n)))
    common = (dev(g), dev(dHq), dev(dHr), dev(X), dev(W), dev(sv), dev(f32(ref["H_pre"])), dev(f32(ref["H_post"])),
              dev(f32(ref["L"])))
    if mode == "accumulate":
        dX0 = store(RNG.standard_normal((N, n, C)), act)
        ob = B.mhc_pre_bwd(*common, alpha=dev(alpha), iters=20, eps=1e-6, dX=dev(dX0), accumulate_dX=True,
                           want_intermediates=True)
        base = h64(dX0)
    else:
        Gp = store(RNG.standard_normal((N, n, C)), act)
        Hrp = f32(O.sinkhorn_fwd(RNG.standard_normal((N, n, n)), 20, 1e-6))
        ob = B.mhc_pre_bwd(*common, alpha=dev(alpha), iters=20, eps=1e-6, want_intermediates=True,
                           post_G=dev(Gp), post_H_res=dev(Hrp))
        base = O.stream_mix_bwd(h64(Gp), h64(X), h64(Hrp))[0]
    torch.cuda.synchronize()
    rb = O.pre_bwd(h64(g), h64(dHq), h64(dHr), h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    assert_mixed("dH_pre", ob["dH_pre"], rb["dH_pre"])
    assert_mixed("dlogits", ob["dlogits"], rb["dL"])
    assert_act("dX", ob["dX"], base + rb["dX"], act)
    aW, aa, ab = _abs_parts_pre(h64(g), h64(dHq), h64(dHr), h64(X), h64(W), h64(alpha), h64(hb))
    assert_tokensum("dW", ob["dW"], rb["dW"], aW, depth=sum_depth("proj", N, C, n=n, act=act))
    assert_tokensum("dalpha", ob["dalpha"], rb["dalpha"], aa, depth=sum_depth("param", N, n=n))
    assert_tokensum("dhbias", ob["dhbias"], rb["dhbias"], ab, depth=sum_depth("param", N, n=n))


def test_general_n_deterministic_and_zero_tokens():
    n, N, C = 8, 50, 296
    X, W, alpha, hb = _proj_inputs(n, "bf16", N, C)
    a = B.mhc_pre_fwd(dev(X), dev(W))
    b = B.mhc_pre_fwd(dev(X), dev(W))
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    Z = torch.zeros(0, 3, 64, dtype=torch.bfloat16, device="cuda")
    Wz = torch.zeros(3 * 64, 15, device="cuda")
    o = B.mhc_pre_fwd(Z, Wz)
    torch.cuda.synchronize()
    assert o["agg"].shape == (0, 64)


@pytest.mark.parametrize("n", [2, 8])
def test_general_n_max_width(n):
    """C = 16384 (the largest width) with a ragged token count: pre forward and the fused
    pre backward with the h_post_bda term, against the oracle."""
    N, C, act = 5, 16384, "bf16"
    log(f"general n max width n={n} N={N} C={C}")
    X, W, alpha, hb = _proj_inputs(n, act, N, C)
    J = n * n + 2 * n
    o = B.mhc_pre_fwd(dev(X), dev(W), dev(alpha), dev(hb), 1e-6, 20, 1e-6)
    torch.cuda.synchronize()
    ref = O.pre_fwd(h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    assert_rel("H_pre", o["H_pre"], ref["H_pre"])
    assert_h_res(o["H_res"], o["H_res_logits"], ref["H_res"], ref["L"], 20, 1e-6,
                 alone=B.mhc_sinkhorn_fwd(o["H_res_logits"], 20, 1e-6))
    assert_act("agg", o["agg"], ref["agg"], act)
    sv = np.zeros((N, B.saved_stride(n)), np.float32)
    sv[:, 0] = ref["r"]; sv[:, 1] = ref["q"]; sv[:, 2:2 + J] = ref["z"]
    g = store(RNG.standard_normal((N, C)), act)
    dHq = f32(RNG.standard_normal((N, n)))
    dHr = f32(RNG.standard_normal((N, n, n)))
    Gp = store(RNG.standard_normal((N, n, C)), act)
    Hrp = f32(O.sinkhorn_fwd(RNG.standard_normal((N, n, n)), 20, 1e-6))
    ob = B.mhc_pre_bwd(dev(g), dev(dHq), dev(dHr), dev(X), dev(W), dev(sv), dev(f32(ref["H_pre"])),
                       dev(f32(ref["H_post"])), dev(f32(ref["L"])), alpha=dev(alpha), iters=20, eps=1e-6,
                       post_G=dev(Gp), post_H_res=dev(Hrp))
    torch.cuda.synchronize()
    rb = O.pre_bwd(h64(g), h64(dHq), h64(dHr), h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    base = O.stream_mix_bwd(h64(Gp), h64(X), h64(Hrp))[0]
    assert_act("dX", ob["dX"], base + rb["dX"], act)
    aW, aa, ab = _abs_parts_pre(h64(g), h64(dHq), h64(dHr), h64(X), h64(W), h64(alpha), h64(hb))
    assert_tokensum("dW", ob["dW"], rb["dW"], aW, depth=sum_depth("proj", N, C, n=n, act=act))
    assert_tokensum("dalpha", ob["dalpha"], rb["dalpha"], aa, depth=sum_depth("param", N, n=n))


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("n,C", [(2, 1032), (2, 8192), (8, 296)])
def test_general_n_per_token_results_batch_invariant(n, C):
    """As for n = 4: the same 37 tokens alone and at rows 700..736 of a 1300-token batch give the
    same bits for every per-token output (sums over tokens excluded)."""
    n_small, n_big, at = 37, 1300, 700
    log(f"general n batch invariance n={n} C={C}")
    act = "bf16"
    Xb, W, alpha, hb = _proj_inputs(n, act, n_big, C)
    Gb = store(RNG.standard_normal((n_big, n, C)), act)
    xb = store(RNG.standard_normal((n_big, C)), act)
    gb = store(RNG.standard_normal((n_big, C)), act)
    bias = store(RNG.standard_normal(C) * 0.1, act)
    dHpb = f32(RNG.standard_normal((n_big, n)))
    dHrb = f32(RNG.standard_normal((n_big, n, n)))
    sl = slice(at, at + n_small)

    def run(X, G, x, g, dHp, dHr):
        r = {}
        o = B.mhc_pre_fwd(dev(X), dev(W), dev(alpha), dev(hb))
        r.update({f"pre_fwd.{k}": v for k, v in o.items()})
        r["sk_bwd"] = B.mhc_sinkhorn_bwd(dev(dHr), o["H_res_logits"])
        r["post_fwd"] = B.mhc_h_post_bda_fwd(dev(X), o["H_res"], o["H_post"], dev(x), dev(bias))
        pdX, pdHr, pdHp, pdx, _ = B.mhc_h_post_bda_bwd(dev(G), dev(X), o["H_res"], o["H_post"], dev(x), dev(bias),
                                                       want_dbias=False)
        r.update({"post_bwd.dX": pdX, "post_bwd.dH_res": pdHr, "post_bwd.dH_post": pdHp, "post_bwd.dx": pdx})
        bw = B.mhc_pre_bwd(dev(g), dev(dHp), dev(dHr), dev(X), dev(W), o["saved"], o["H_pre"], o["H_post"],
                           o["H_res_logits"], alpha=dev(alpha), want_intermediates=True, post_G=dev(G),
                           post_H_res=o["H_res"])
        r.update({"pre_bwd.dX": bw["dX"], "pre_bwd.dH_pre": bw["dH_pre"], "pre_bwd.dlogits": bw["dlogits"]})
        torch.cuda.synchronize()
        return r

    big = run(Xb, Gb, xb, gb, dHpb, dHrb)
    small = run(*(np.ascontiguousarray(a[sl]) for a in (Xb, Gb, xb, gb, dHpb, dHrb)))
    for k, v in small.items():
        assert torch.equal(_bits(v), _bits(big[k][sl])), f"{k}: per-token result depends on the batch"
