"""GPU parity: each libmhc entry point against the fp64 oracle, element by element.

Inputs are seeded synthetic arrays (mhc_hyper_connection_proj_amd.synth) or
oracle outputs rounded to their storage type; nothing fed to the oracle comes
from the GPU.  Sizes span several MFMA/workgroup tiles and ragged tails.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (assert_act, assert_h_res, assert_mixed, assert_rel, assert_tokensum, dev, h64, log,
                      pre_bwd_abs_parts, proj_bwd_abs_parts, sinkhorn_rtol, sum_depth)
from mhc_hyper_connection_proj_amd import binding as B
from mhc_hyper_connection_proj_amd import synth

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(7)


def f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def store(a64, act):
    """float64 -> storage array (bf16 bits or float32), rounding once."""
    return O.round_f64_to_bf16_bits(a64) if act == "bf16" else f32(a64)


# ----------------------------------------------------------------- Sinkhorn
@pytest.mark.parametrize("count,iters,eps,std", [
    (1, 20, 1e-6, 1.0), (5000, 20, 1e-6, 1.0), (777, 20, 1e-6, 3.4), (300, 0, 1e-6, 1.0),
    (300, 1, 1e-6, 1.0), (300, 45, 1e-6, 1.0), (300, 7, 0.25, 1.0), (300, 20, 0.0, 1.0),
    # long runs: the backward replays 20-iteration segments, rebuilding each half-step's input as M' d
    (1000, 100, 1e-6, 1.0), (1000, 150, 0.25, 1.0), (1000, 200, 1e-6, 1.0), (1000, 200, 1e-6, 2.0)])
def test_sinkhorn_fwd_bwd(count, iters, eps, std):
    log(f"sinkhorn count={count} iters={iters} eps={eps} std={std}")
    L = f32(RNG.standard_normal((count, 4, 4)) * std)
    dH = f32(RNG.standard_normal((count, 4, 4)))
    H = B.mhc_sinkhorn_fwd(dev(L), iters, eps)
    dL = B.mhc_sinkhorn_bwd(dev(dH), dev(L), iters, eps)
    torch.cuda.synchronize()
    oH, odL = O.sinkhorn_fwd(h64(L), iters, eps), O.sinkhorn_bwd(h64(dH), h64(L), iters, eps)
    rms = np.sqrt(np.mean(odL * odL))
    log(f"  worst error / 1e-5 bound: H_res {np.max(np.abs(h64(H) - oH) / (1e-5 * np.abs(oH))):.3f}, "
        f"dlogits {np.max(np.abs(h64(dL) - odL) / (1e-5 * (np.abs(odL) + rms))):.3f}")
    assert_rel("H_res", H, oH)
    assert_mixed("dlogits", dL, odL, rtol=sinkhorn_rtol(iters, grad=True, n=4))


def test_sinkhorn_batched_workload_full():
    w = synth.WORKLOADS["sinkhorn_batched"]
    log(f"sinkhorn full workload count={w.tokens}")
    L = synth.tensor(w, "L")
    dH = synth.tensor(w, "dH")
    H = B.mhc_sinkhorn_fwd(dev(L), w.iters, w.eps)
    dL = B.mhc_sinkhorn_bwd(dev(dH), dev(L), w.iters, w.eps)
    torch.cuda.synchronize()
    assert_rel("H_res", H, O.sinkhorn_fwd(h64(L), w.iters, w.eps))
    assert_mixed("dlogits", dL, O.sinkhorn_bwd(h64(dH), h64(L), w.iters, w.eps))


# ----------------------------------------------------------------- h_aggregate
SHAPES = [("bf16", 1, 256), ("bf16", 37, 296), ("bf16", 9, 4096), ("bf16", 5, 7168),
          ("f32", 64, 256), ("f32", 11, 1032), ("bf16", 3, 8), ("bf16", 2, 16384), ("f32", 2, 12288)]


@pytest.mark.parametrize("act,N,C", SHAPES)
def test_h_aggregate(act, N, C):
    log(f"h_aggregate act={act} N={N} C={C}")
    X = store(RNG.standard_normal((N, 4, C)), act)
    Hp = f32(1 / (1 + np.exp(-RNG.standard_normal((N, 4)))))
    g = store(RNG.standard_normal((N, C)), act)
    dX0 = store(RNG.standard_normal((N, 4, C)), act)
    Xd = dev(X)
    out = B.mhc_h_aggregate_fwd(Xd, dev(Hp))
    dX, dH = B.mhc_h_aggregate_bwd(dev(g), Xd, dev(Hp))
    dXa, _ = B.mhc_h_aggregate_bwd(dev(g), Xd, dev(Hp), dX=dev(dX0), accumulate_dX=True)
    torch.cuda.synchronize()
    assert_act("agg", out, O.h_aggregate_fwd(h64(X), h64(Hp)), act)
    odX, odH = O.h_aggregate_bwd(h64(g), h64(X), h64(Hp))
    assert_act("dX", dX, odX, act)
    assert_act("dX accumulated", dXa, h64(dX0) + odX, act)
    assert_mixed("dH_pre", dH, odH)


def test_h_aggregate_one_hot_exact():
    N, C = 40, 7168
    X = synth.f32_to_bf16_bits(RNG.standard_normal((N, 4, C)).astype(np.float32))
    sel = RNG.integers(0, 4, N)
    Hp = f32(np.eye(4)[sel])
    out = B.mhc_h_aggregate_fwd(dev(X), dev(Hp))
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, X[np.arange(N), sel])


# ----------------------------------------------------------------- h_post_bda
@pytest.mark.parametrize("act,N,C,bias", [
    ("bf16", 1, 256, True), ("bf16", 37, 296, True), ("bf16", 50, 4096, True), ("bf16", 21, 7168, False),
    ("f32", 64, 256, True), ("f32", 17, 1032, False), ("bf16", 33, 8, True), ("bf16", 3, 16384, True),
    ("bf16", 9, 5120, False), ("bf16", 6, 6144, True), ("bf16", 4, 8192, False), ("bf16", 5, 7168, True),
    # with dbias, bf16 rows of up to 1024 8-channel groups take the one-token-ahead kernel (C = 8192: a
    # 1024-thread workgroup); C = 8200 is the first width that falls back to the four-groups-per-thread form
    ("bf16", 19, 8192, True), ("bf16", 7, 8200, True)])
def test_h_post_bda(act, N, C, bias):
    log(f"h_post_bda act={act} N={N} C={C} bias={bias}")
    X = store(RNG.standard_normal((N, 4, C)), act)
    G = store(RNG.standard_normal((N, 4, C)), act)
    x = store(RNG.standard_normal((N, C)), act)
    b = store(RNG.standard_normal(C) * 0.1, act) if bias else None
    Hr = f32(O.sinkhorn_fwd(RNG.standard_normal((N, 4, 4)), 20, 1e-6))
    Hp = f32(2 / (1 + np.exp(-RNG.standard_normal((N, 4)))))
    out = B.mhc_h_post_bda_fwd(dev(X), dev(Hr), dev(Hp), dev(x), dev(b) if bias else None)
    dX, dHr, dHp, dx, db = B.mhc_h_post_bda_bwd(dev(G), dev(X), dev(Hr), dev(Hp), dev(x),
                                                dev(b) if bias else None)
    torch.cuda.synchronize()
    bb = h64(b) if bias else None
    assert_act("out", out, O.h_post_bda_fwd(h64(X), h64(Hr), h64(Hp), h64(x), bb), act)
    odX, odHr, odHp, odx, odb = O.h_post_bda_bwd(h64(G), h64(X), h64(Hr), h64(Hp), h64(x), bb)
    assert_act("dX", dX, odX, act)
    assert_mixed("dH_res", dHr, odHr)
    assert_mixed("dH_post", dHp, odHp)
    assert_act("dx", dx, odx, act)
    if bias:
        assert_tokensum("dbias", db, odb, np.abs(odx).sum(axis=0), act, sum_depth("rows", N))
    else:
        assert db is None
    # without dX (the pre backward forms it), also without dbias: the other
    # outputs to the same rules (another kernel may serve this case, so the
    # fp32 summation order, and the last bits, can differ from the run above)
    for want_db, want_dX in (((True, False), (False, False), (False, True)) if bias else ((False, False),)):
        nX, nHr, nHp, ndx, ndb = B.mhc_h_post_bda_bwd(dev(G), dev(X), dev(Hr), dev(Hp), dev(x),
                                                      dev(b) if bias else None, want_dbias=want_db, want_dX=want_dX)
        torch.cuda.synchronize()
        if want_dX:
            assert_act("dX (no dbias)", nX, odX, act)
        else:
            assert nX is None
        assert_mixed("dH_res (no dX)", nHr, odHr)
        assert_mixed("dH_post (no dX)", nHp, odHp)
        assert_act("dx (no dX)", ndx, odx, act)
        if want_db:
            assert_tokensum("dbias (no dX)", ndb, odb, np.abs(odx).sum(axis=0), act, sum_depth("rows", N))


# ----------------------------------------------------------------- stream mix / distribute, shared-row aggregate
VARIANT_SHAPES = [("bf16", 1, 8), ("bf16", 37, 296), ("bf16", 50, 4096), ("f32", 17, 1032), ("bf16", 21, 7168),
                  ("bf16", 3, 16384)]


@pytest.mark.parametrize("act,N,C", VARIANT_SHAPES)
def test_stream_mix(act, N, C):
    log(f"stream mix act={act} N={N} C={C}")
    X = store(RNG.standard_normal((N, 4, C)), act)
    G = store(RNG.standard_normal((N, 4, C)), act)
    M = f32(RNG.standard_normal((N, 4, 4)))
    out = B.mhc_stream_mix_fwd(dev(X), dev(M))
    dX, dM = B.mhc_stream_mix_bwd(dev(G), dev(X), dev(M))
    torch.cuda.synchronize()
    assert_act("out", out, O.stream_mix_fwd(h64(X), h64(M)), act)
    odX, odM = O.stream_mix_bwd(h64(G), h64(X), h64(M))
    assert_act("dX", dX, odX, act)
    assert_mixed("dM", dM, odM)


@pytest.mark.parametrize("act,N,C", VARIANT_SHAPES)
def test_stream_distribute(act, N, C):
    log(f"stream distribute act={act} N={N} C={C}")
    x = store(RNG.standard_normal((N, C)), act)
    G = store(RNG.standard_normal((N, 4, C)), act)
    Hp = f32(RNG.standard_normal((N, 4)))
    out = B.mhc_stream_distribute_fwd(dev(x), dev(Hp))
    dx, dH = B.mhc_stream_distribute_bwd(dev(G), dev(x), dev(Hp))
    torch.cuda.synchronize()
    assert_act("out", out, O.stream_distribute_fwd(h64(x), h64(Hp)), act)
    odx, odH = O.stream_distribute_bwd(h64(G), h64(x), h64(Hp))
    assert_act("dx", dx, odx, act)
    assert_mixed("dH_post", dH, odH)


@pytest.mark.parametrize("act,N,C", VARIANT_SHAPES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_h_aggregate_static(act, N, C, accumulate):
    log(f"h_aggregate static act={act} N={N} C={C} accumulate={accumulate}")
    X = store(RNG.standard_normal((N, 4, C)), act)
    g = store(RNG.standard_normal((N, C)), act)
    h = f32(RNG.standard_normal(4))
    out = B.mhc_h_aggregate_static_fwd(dev(X), dev(h))
    dX0 = store(RNG.standard_normal((N, 4, C)), act) if accumulate else None
    dX, dH = B.mhc_h_aggregate_static_bwd(dev(g), dev(X), dev(h), dX=dev(dX0) if accumulate else None,
                                          accumulate_dX=accumulate)
    torch.cuda.synchronize()
    assert_act("agg", out, O.h_aggregate_static_fwd(h64(X), h64(h)), act)
    odX, odH = O.h_aggregate_static_bwd(h64(g), h64(X), h64(h))
    assert_act("dX", dX, odX + (h64(dX0) if accumulate else 0.0), act)
    parts = np.abs(O.h_aggregate_bwd(h64(g), h64(X), np.broadcast_to(h64(h), (N, 4)).copy())[1]).sum(axis=0)
    assert_tokensum("dH_pre", dH, odH, parts, depth=sum_depth("hpre", N))


def test_variants_zero_tokens():
    X = torch.empty(0, 4, 64, dtype=torch.bfloat16, device="cuda")
    dX, dH = B.mhc_h_aggregate_static_bwd(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"), X,
                                          torch.ones(4, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(dH.cpu(), torch.zeros(4))
    assert B.mhc_stream_mix_fwd(X, torch.empty(0, 4, 4, device="cuda")).shape == X.shape


def test_h_post_bda_identity_h_res_exact_bf16():
    # H_res = I and H_post = 0: out must reproduce the residual bit for bit
    N, C = 19, 4096
    X = synth.f32_to_bf16_bits(RNG.standard_normal((N, 4, C)).astype(np.float32))
    x = synth.f32_to_bf16_bits(RNG.standard_normal((N, C)).astype(np.float32))
    Hr = f32(np.broadcast_to(np.eye(4), (N, 4, 4)))
    out = B.mhc_h_post_bda_fwd(dev(X), dev(Hr), dev(np.zeros((N, 4), np.float32)), dev(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), X)


# ----------------------------------------------------------------- projection
# 1030 tokens at C = 4096 and 8192: five token blocks, so the staggered projection walk (rows a multiple of
# 16 KB apart) starts at every one of its four sub-slices
PROJ = [("f32", 64, 256), ("bf16", 37, 296), ("bf16", 70, 4096), ("bf16", 67, 7168),
        ("bf16", 5, 8), ("f32", 33, 1032), ("bf16", 129, 1024), ("bf16", 33, 16384),
        ("bf16", 1030, 4096), ("bf16", 1030, 8192)]


def _proj_inputs(act, N, C, zero_row=True):
    X = store(RNG.standard_normal((N, 4, C)), act)
    if zero_row and N > 3:
        X[2] = 0
    W = f32(RNG.standard_normal((4 * C, 24)) * 0.02)
    alpha = f32([1.3, 0.7, 1.1])
    hb = f32(RNG.standard_normal(24) * 0.1)
    return X, W, alpha, hb


@pytest.mark.parametrize("act,N,C", PROJ)
def test_proj_rms_h_fwd(act, N, C):
    log(f"proj_rms_h fwd act={act} N={N} C={C}")
    X, W, alpha, hb = _proj_inputs(act, N, C)
    Hp, Hq, L, saved = B.mhc_proj_rms_h(dev(X), dev(W), dev(alpha), dev(hb), 1e-6)
    torch.cuda.synchronize()
    p = O.proj_rms_h(h64(X), h64(W), h64(alpha), h64(hb), 1e-6)
    # upstream quantities first, so a failure names the first diverging value
    s = h64(saved)
    assert_rel("q", s[:, 1], p.q)
    assert_rel("r", s[:, 0], p.r)
    assert_mixed("z", s[:, 2:26], p.z)
    np.testing.assert_array_equal(s[:, 26:], 0.0)
    assert_mixed("logits", L, p.L)
    assert_rel("H_pre", Hp, p.H_pre)
    assert_rel("H_post", Hq, p.H_post)


@pytest.mark.parametrize("N,C", [(37, 296), (70, 4096), (67, 7168), (5, 8), (129, 1024), (33, 16384), (300, 64)])
def test_proj_rms_h_fma(N, C):
    """The VALU (FMA) form of the forward projection, kept as the MFMA choice's comparison point."""
    log(f"proj_rms_h fma N={N} C={C}")
    X, W, alpha, hb = _proj_inputs("bf16", N, C)
    Hp, Hq, L, saved = B.mhc_proj_rms_h_fma(dev(X), dev(W), dev(alpha), dev(hb), 1e-6)
    torch.cuda.synchronize()
    p = O.proj_rms_h(h64(X), h64(W), h64(alpha), h64(hb), 1e-6)
    s = h64(saved)
    assert_rel("q", s[:, 1], p.q)
    assert_rel("r", s[:, 0], p.r)
    assert_mixed("z", s[:, 2:26], p.z)
    np.testing.assert_array_equal(s[:, 26:], 0.0)
    assert_mixed("logits", L, p.L)
    assert_rel("H_pre", Hp, p.H_pre)
    assert_rel("H_post", Hq, p.H_post)


@pytest.mark.parametrize("act,N,C", PROJ)
def test_proj_rms_h_bwd(act, N, C):
    log(f"proj_rms_h bwd act={act} N={N} C={C}")
    X, W, alpha, hb = _proj_inputs(act, N, C)
    p = O.proj_rms_h(h64(X), h64(W), h64(alpha), h64(hb), 1e-6)
    saved = np.zeros((N, 32), np.float32)
    saved[:, 0] = p.r; saved[:, 1] = p.q; saved[:, 2:26] = p.z
    Hp, Hq = f32(p.H_pre), f32(p.H_post)
    dHp = f32(RNG.standard_normal((N, 4))); dHq = f32(RNG.standard_normal((N, 4)))
    dL = f32(RNG.standard_normal((N, 4, 4)))
    dX0 = store(RNG.standard_normal((N, 4, C)), act)
    args = (dev(X), dev(W), dev(saved), dev(Hp), dev(Hq), dev(dHp), dev(dHq), dev(dL))
    dX, dW, da, db = B.mhc_proj_rms_h_bwd(*args, alpha=dev(alpha))
    dXa, _, _, _ = B.mhc_proj_rms_h_bwd(*args, alpha=dev(alpha), dX=dev(dX0), accumulate_dX=True,
                                        want_dW=False, want_dalpha=False, want_dhbias=False)
    torch.cuda.synchronize()
    odX, odW, oda, odb = O.proj_rms_h_bwd(h64(X), h64(W), h64(dHp), h64(dHq), h64(dL), h64(alpha), h64(hb), 1e-6)
    assert_act("dX", dX, odX, act)
    assert_act("dX accumulated", dXa, h64(dX0) + odX, act)
    aW, aa, ab = proj_bwd_abs_parts(h64(X), h64(W), h64(dHp), h64(dHq), h64(dL), h64(alpha), h64(hb), 1e-6)
    assert_tokensum("dW", dW, odW, aW, depth=sum_depth("proj", N, C, act=act))
    assert_tokensum("dalpha", da, oda, aa, depth=sum_depth("param", N))
    assert_tokensum("dhbias", db, odb, ab, depth=sum_depth("param", N))


# ----------------------------------------------------------------- fused pre pass
@pytest.mark.parametrize("mode", ["accumulate", "post"])
@pytest.mark.parametrize("act,N,C", [("f32", 64, 256), ("bf16", 37, 296), ("bf16", 66, 7168), ("bf16", 130, 4096),
                                     ("bf16", 1000, 2048), ("bf16", 520, 4096), ("bf16", 33, 16384), ("bf16", 1, 8),
                                     ("bf16", 17, 72)])
def test_pre_fwd_bwd(act, N, C, mode):
    log(f"pre fwd/bwd act={act} N={N} C={C} mode={mode}")
    X, W, alpha, hb = _proj_inputs(act, N, C)
    o = B.mhc_pre_fwd(dev(X), dev(W), dev(alpha), dev(hb), 1e-6, 20, 1e-6)
    torch.cuda.synchronize()
    ref = O.pre_fwd(h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    assert_rel("H_pre", o["H_pre"], ref["H_pre"])
    assert_rel("H_post", o["H_post"], ref["H_post"])
    assert_mixed("logits", o["H_res_logits"], ref["L"])
    assert_h_res(o["H_res"], o["H_res_logits"], ref["H_res"], ref["L"], 20, 1e-6,
                 alone=B.mhc_sinkhorn_fwd(o["H_res_logits"], 20, 1e-6))
    assert_act("agg", o["agg"], ref["agg"], act)
    # backward from oracle-produced forward state
    saved = np.zeros((N, 32), np.float32)
    saved[:, 0] = ref["r"]; saved[:, 1] = ref["q"]; saved[:, 2:26] = ref["z"]
    g = store(RNG.standard_normal((N, C)), act)
    dHq = f32(RNG.standard_normal((N, 4)))
    dHr = f32(RNG.standard_normal((N, 4, 4)))
    if mode == "accumulate":  # the h_post_bda dX comes in materialised
        dX0 = store(RNG.standard_normal((N, 4, C)), act)
        ob = B.mhc_pre_bwd(dev(g), dev(dHq), dev(dHr), dev(X), dev(W), dev(saved), dev(f32(ref["H_pre"])),
                           dev(f32(ref["H_post"])), dev(f32(ref["L"])), alpha=dev(alpha), iters=20, eps=1e-6,
                           dX=dev(dX0), accumulate_dX=True, want_intermediates=True)
        base = h64(dX0)
    else:  # the h_post_bda dX term formed here from its G and H_res
        Gp = store(RNG.standard_normal((N, 4, C)), act)
        Hrp = f32(O.sinkhorn_fwd(RNG.standard_normal((N, 4, 4)), 20, 1e-6))
        ob = B.mhc_pre_bwd(dev(g), dev(dHq), dev(dHr), dev(X), dev(W), dev(saved), dev(f32(ref["H_pre"])),
                           dev(f32(ref["H_post"])), dev(f32(ref["L"])), alpha=dev(alpha), iters=20, eps=1e-6,
                           want_intermediates=True, post_G=dev(Gp), post_H_res=dev(Hrp))
        zeros = np.zeros((N, 4)); zc = np.zeros((N, C))
        base = O.h_post_bda_bwd(h64(Gp), h64(X), h64(Hrp), zeros, zc)[0]
    torch.cuda.synchronize()
    rb = O.pre_bwd(h64(g), h64(dHq), h64(dHr), h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    assert_mixed("dH_pre", ob["dH_pre"], rb["dH_pre"])
    assert_mixed("dlogits", ob["dlogits"], rb["dL"])
    assert_act("dX", ob["dX"], base + rb["dX"], act)
    aW, aa, ab = pre_bwd_abs_parts(h64(g), h64(dHq), h64(dHr), h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    assert_tokensum("dW", ob["dW"], rb["dW"], aW, depth=sum_depth("proj", N, C, act=act))
    assert_tokensum("dalpha", ob["dalpha"], rb["dalpha"], aa, depth=sum_depth("param", N))
    assert_tokensum("dhbias", ob["dhbias"], rb["dhbias"], ab, depth=sum_depth("param", N))


@pytest.mark.parametrize("act,N,C", [("bf16", 37, 296), ("bf16", 66, 7168), ("bf16", 130, 4096)])
def test_pre_bwd_post_term_accumulate_no_dw(act, N, C):
    # the h_post_bda dX term formed in the pass and the result added onto a given dX, with dW not
    # requested: the remaining variants of the fused dX/dW kernel (the other tests write dX fresh
    # and always take dW)
    log(f"pre bwd post term + accumulate, no dW act={act} N={N} C={C}")
    X, W, alpha, hb = _proj_inputs(act, N, C)
    ref = O.pre_fwd(h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    saved = np.zeros((N, 32), np.float32)
    saved[:, 0] = ref["r"]; saved[:, 1] = ref["q"]; saved[:, 2:26] = ref["z"]
    g = store(RNG.standard_normal((N, C)), act)
    dHq = f32(RNG.standard_normal((N, 4)))
    dHr = f32(RNG.standard_normal((N, 4, 4)))
    dX0 = store(RNG.standard_normal((N, 4, C)), act)
    Gp = store(RNG.standard_normal((N, 4, C)), act)
    Hrp = f32(O.sinkhorn_fwd(RNG.standard_normal((N, 4, 4)), 20, 1e-6))
    ob = B.mhc_pre_bwd(dev(g), dev(dHq), dev(dHr), dev(X), dev(W), dev(saved), dev(f32(ref["H_pre"])),
                       dev(f32(ref["H_post"])), dev(f32(ref["L"])), alpha=dev(alpha), iters=20, eps=1e-6,
                       dX=dev(dX0), accumulate_dX=True, post_G=dev(Gp), post_H_res=dev(Hrp), want_dW=False)
    torch.cuda.synchronize()
    assert ob["dW"] is None
    zeros = np.zeros((N, 4)); zc = np.zeros((N, C))
    post = O.h_post_bda_bwd(h64(Gp), h64(X), h64(Hrp), zeros, zc)[0]
    rb = O.pre_bwd(h64(g), h64(dHq), h64(dHr), h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    assert_act("dX", ob["dX"], h64(dX0) + post + rb["dX"], act)
    _, aa, ab = pre_bwd_abs_parts(h64(g), h64(dHq), h64(dHr), h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    assert_tokensum("dalpha", ob["dalpha"], rb["dalpha"], aa, depth=sum_depth("param", N))
    assert_tokensum("dhbias", ob["dhbias"], rb["dhbias"], ab, depth=sum_depth("param", N))


@pytest.mark.parametrize("iters,eps", [(100, 1e-6), (200, 1e-6), (150, 0.25)])
def test_pre_fwd_bwd_long_iterations(iters, eps):
    """The fused pre pass runs its Sinkhorn in the quad layout (finalize forward, per-token backward):
    long iteration counts, against the oracle at the iteration-count rule."""
    N, C, act = 37, 296, "bf16"
    log(f"pre fwd/bwd long iterations iters={iters} eps={eps}")
    X, W, alpha, hb = _proj_inputs(act, N, C)
    o = B.mhc_pre_fwd(dev(X), dev(W), dev(alpha), dev(hb), 1e-6, iters, eps)
    torch.cuda.synchronize()
    ref = O.pre_fwd(h64(X), h64(W), h64(alpha), h64(hb), 1e-6, iters, eps)
    assert_mixed("logits", o["H_res_logits"], ref["L"])
    assert_h_res(o["H_res"], o["H_res_logits"], ref["H_res"], ref["L"], iters, eps,
                 alone=B.mhc_sinkhorn_fwd(o["H_res_logits"], iters, eps))
    saved = np.zeros((N, 32), np.float32)
    saved[:, 0] = ref["r"]; saved[:, 1] = ref["q"]; saved[:, 2:26] = ref["z"]
    g = store(RNG.standard_normal((N, C)), act)
    dHq, dHr = f32(RNG.standard_normal((N, 4))), f32(RNG.standard_normal((N, 4, 4)))
    ob = B.mhc_pre_bwd(dev(g), dev(dHq), dev(dHr), dev(X), dev(W), dev(saved), dev(f32(ref["H_pre"])),
                       dev(f32(ref["H_post"])), dev(f32(ref["L"])), alpha=dev(alpha), iters=iters, eps=eps,
                       want_intermediates=True)
    alone = B.mhc_sinkhorn_bwd(dev(dHr), dev(f32(ref["L"])), iters, eps)
    torch.cuda.synchronize()
    odL = O.sinkhorn_bwd(h64(dHr), h64(f32(ref["L"])), iters, eps)
    rms = np.sqrt(np.mean(odL * odL))
    log(f"  dlogits worst error / 1e-5 bound: fused {np.max(np.abs(h64(ob['dlogits']) - odL) / (1e-5 * (np.abs(odL) + rms))):.3f}"
        f", standalone {np.max(np.abs(h64(alone) - odL) / (1e-5 * (np.abs(odL) + rms))):.3f}")
    assert_mixed("dlogits (fused)", ob["dlogits"], odL, rtol=sinkhorn_rtol(iters, grad=True, n=4))
    assert_mixed("dlogits (standalone)", alone, odL, rtol=sinkhorn_rtol(iters, grad=True, n=4))


# ----------------------------------------------------------------- measurement hook
def test_kernel_events_hook_times_dxdw_and_changes_nothing():
    from mhc_hyper_connection_proj_amd import _lib as L
    N, C = 300, 1024
    log(f"kernel events hook N={N} C={C}")
    X, W, alpha, hb = _proj_inputs("bf16", N, C)
    ref = O.pre_fwd(h64(X), h64(W), h64(alpha), h64(hb), 1e-6, 20, 1e-6)
    saved = np.zeros((N, 32), np.float32)
    saved[:, 0] = ref["r"]; saved[:, 1] = ref["q"]; saved[:, 2:26] = ref["z"]
    g = store(RNG.standard_normal((N, C)), "bf16")
    dHq, dHr = f32(RNG.standard_normal((N, 4))), f32(RNG.standard_normal((N, 4, 4)))
    args = (dev(g), dev(dHq), dev(dHr), dev(X), dev(W), dev(saved), dev(f32(ref["H_pre"])), dev(f32(ref["H_post"])),
            dev(f32(ref["L"])))
    plain = B.mhc_pre_bwd(*args, alpha=dev(alpha), iters=20, eps=1e-6)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record(stream)
    lib = L.lib()
    L.check(lib.mhc_set_kernel_events(L.MHC_KERNEL_PROJ_BWD_DXDW, ev[0]._as_parameter_, ev[1]._as_parameter_))
    try:
        hooked = B.mhc_pre_bwd(*args, alpha=dev(alpha), iters=20, eps=1e-6)
    finally:
        L.check(lib.mhc_set_kernel_events(L.MHC_KERNEL_NONE, None, None))
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0.0
    for k in ("dX", "dW", "dalpha", "dhbias"):
        assert torch.equal(plain[k], hooked[k]), k


# ----------------------------------------------------------------- edge cases
def test_zero_tokens_is_noop_and_zero_param_grads():
    C = 64
    X = torch.empty(0, 4, C, dtype=torch.bfloat16, device="cuda")
    W = torch.randn(4 * C, 24, device="cuda")
    e = torch.empty(0, 4, device="cuda")
    o = B.mhc_pre_bwd(torch.empty(0, C, dtype=torch.bfloat16, device="cuda"), e, torch.empty(0, 4, 4, device="cuda"),
                      X, W, torch.empty(0, 32, device="cuda"), e, e, torch.empty(0, 4, 4, device="cuda"))
    torch.cuda.synchronize()
    assert o["dW"].abs().max().item() == 0.0
    assert o["dalpha"].abs().max().item() == 0.0 and o["dhbias"].abs().max().item() == 0.0
    assert B.mhc_sinkhorn_fwd(torch.empty(0, 4, 4, device="cuda")).numel() == 0


def test_deterministic_bitwise():
    act, N, C = "bf16", 96, 4096
    X, W, alpha, hb = _proj_inputs(act, N, C)
    G = store(RNG.standard_normal((N, 4, C)), act)
    x = store(RNG.standard_normal((N, C)), act)
    b = store(RNG.standard_normal(C) * 0.1, act)
    outs = []
    for _ in range(2):
        o = B.mhc_pre_fwd(dev(X), dev(W), dev(alpha), dev(hb))
        pb = B.mhc_h_post_bda_bwd(dev(G), dev(X), o["H_res"], o["H_post"], dev(x), dev(b))
        bw = B.mhc_pre_bwd(o["agg"], pb[2], pb[1], dev(X), dev(W), o["saved"], o["H_pre"], o["H_post"],
                           o["H_res_logits"], alpha=dev(alpha))
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (*o.values(), *[p for p in pb if p is not None], *bw.values())])
    for a, b2 in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a, b2.view(torch.uint8)
                           if b2.dtype == torch.bfloat16 else b2)


def _bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("act,C", [("bf16", 2048), ("bf16", 4096), ("f32", 256)])
def test_per_token_results_batch_invariant(act, C):
    """Every per-token output is a function of that token's inputs alone, bit for bit: the same
    37 tokens computed as a batch of their own and at rows 700..736 of a 1300-token batch (other
    token blocks, split-K slices, MFMA sub-tiles and workgroup counts) give identical bits.
    Sums over tokens (dW, dalpha, dhbias, dbias) are excluded: they depend on the batch."""
    n_small, n_big, at = 37, 1300, 700
    log(f"batch invariance act={act} C={C}")
    Xb, W, alpha, hb = _proj_inputs(act, n_big, C)
    Gb = store(RNG.standard_normal((n_big, 4, C)), act)
    xb = store(RNG.standard_normal((n_big, C)), act)
    gb = store(RNG.standard_normal((n_big, C)), act)
    bias = store(RNG.standard_normal(C) * 0.1, act)
    dHpb = f32(RNG.standard_normal((n_big, 4)))
    dHrb = f32(RNG.standard_normal((n_big, 4, 4)))
    sl = slice(at, at + n_small)

    def run(X, G, x, g, dHp, dHr):
        r = {}
        o = B.mhc_pre_fwd(dev(X), dev(W), dev(alpha), dev(hb))
        r.update({f"pre_fwd.{k}": v for k, v in o.items()})
        Hp, Hq, L, sv = B.mhc_proj_rms_h(dev(X), dev(W), dev(alpha), dev(hb))
        r.update({"proj.H_pre": Hp, "proj.H_post": Hq, "proj.L": L, "proj.saved": sv})
        r["sk_fwd"] = B.mhc_sinkhorn_fwd(o["H_res_logits"])
        r["sk_bwd"] = B.mhc_sinkhorn_bwd(dev(dHr), o["H_res_logits"])
        r["agg_fwd"] = B.mhc_h_aggregate_fwd(dev(X), o["H_pre"])
        adX, adH = B.mhc_h_aggregate_bwd(dev(g), dev(X), o["H_pre"])
        r.update({"agg_bwd.dX": adX, "agg_bwd.dH": adH})
        r["post_fwd"] = B.mhc_h_post_bda_fwd(dev(X), o["H_res"], o["H_post"], dev(x), dev(bias))
        pdX, pdHr, pdHp, pdx, _ = B.mhc_h_post_bda_bwd(dev(G), dev(X), o["H_res"], o["H_post"], dev(x), dev(bias),
                                                       want_dbias=False)
        r.update({"post_bwd.dX": pdX, "post_bwd.dH_res": pdHr, "post_bwd.dH_post": pdHp, "post_bwd.dx": pdx})
        pjdX = B.mhc_proj_rms_h_bwd(dev(X), dev(W), o["saved"], o["H_pre"], o["H_post"], dev(dHp), dev(dHp),
                                    dev(dHr), alpha=dev(alpha))[0]
        r["proj_bwd.dX"] = pjdX
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


def test_invalid_arguments_raise():
    X = torch.zeros(4, 9, 64, dtype=torch.bfloat16, device="cuda")  # n = 9 > 8
    with pytest.raises(B._lib.MhcError) as e:
        B.mhc_h_aggregate_fwd(X, torch.zeros(4, 9, device="cuda"))
    assert e.value.name == "MHC_ERR_UNSUPPORTED"
