"""The tiny forward chain exactly as stated for this path, on the GPU, with its backward.

Workload (synth "tiny_chain"): B=1, T=64, n=4, C=256; fp32 residual N(0,1) [64, 4, 256]; projection
weight fp32 N(0, 0.02^2) [1024, 24]; RMS eps 1e-6; H_pre = sigmoid, H_post = 2 sigmoid (alpha = 1,
no bias of H: the NULL defaults); H_res = Sinkhorn(exp(logits)), 20 iterations, eps 1e-6;
h_aggregate; then h_post_bda with x N(0,1) [64, 256] and bias N(0, 0.1^2) [256], both drawn
independently of agg.  The backward takes independent N(0,1) upstream gradients: G [64, 4, 256] for
the h_post_bda output and g [64, 256] for agg.

Each step is compared with the oracle boundary by boundary (the oracle fed the values the GPU
stored for that step's inputs), and the forward chain end to end (the oracle run from the
synthetic inputs alone) under the first-order bound of the errors it carries from H_res and H_post.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (assert_act, assert_h_res, assert_mixed, assert_rel, assert_tokensum, dev, h64,
                      h_res_chain_bound, log, pre_bwd_abs_parts, sum_depth, _report)
from mhc_hyper_connection_proj_amd import binding as B
from mhc_hyper_connection_proj_amd import synth

pytestmark = pytest.mark.gpu


def test_tiny_chain_as_stated():
    w = synth.WORKLOADS["tiny_chain"]
    N, n, C = w.tokens, w.n, w.C
    log(f"tiny chain as stated: N={N} n={n} C={C} act={w.act}")
    X, W = synth.tensor(w, "X"), synth.tensor(w, "W")
    x, bias = synth.tensor(w, "x"), synth.tensor(w, "bias")
    G, g = synth.tensor(w, "G"), synth.tensor(w, "dy")
    assert X.dtype == np.float32 and X.shape == (N, n, C) and W.shape == (n * C, n * n + 2 * n)

    f = B.mhc_pre_fwd(dev(X), dev(W), None, None, w.rms_eps, w.iters, w.eps)
    out = B.mhc_h_post_bda_fwd(dev(X), f["H_res"], f["H_post"], dev(x), dev(bias))
    dXp, dHr, dHp, dx, dbias = B.mhc_h_post_bda_bwd(dev(G), dev(X), f["H_res"], f["H_post"], dev(x), dev(bias))
    bw = B.mhc_pre_bwd(dev(g), dHp, dHr, dev(X), dev(W), f["saved"], f["H_pre"], f["H_post"], f["H_res_logits"],
                       iters=w.iters, eps=w.eps, dX=dXp.clone(), accumulate_dX=True, want_intermediates=True)
    torch.cuda.synchronize()
    X64, W64, x64, b64, G64, g64 = (h64(a) for a in (X, W, x, bias, G, g))

    # step 1-3: the pre forward against the oracle on the synthetic inputs
    ref = O.pre_fwd(X64, W64, None, None, w.rms_eps, w.iters, w.eps)
    sv = h64(f["saved"])
    assert_rel("r", sv[:, 0], ref["r"])
    assert_rel("q", sv[:, 1], ref["q"])
    assert_mixed("z", sv[:, 2:26], ref["z"])
    assert_rel("H_pre", f["H_pre"], ref["H_pre"])
    assert_rel("H_post", f["H_post"], ref["H_post"])
    assert_mixed("logits", f["H_res_logits"], ref["L"])
    assert_h_res(f["H_res"], f["H_res_logits"], ref["H_res"], ref["L"], w.iters, w.eps,
                 alone=B.mhc_sinkhorn_fwd(f["H_res_logits"], w.iters, w.eps))
    assert_act("agg", f["agg"], ref["agg"], w.act)

    # step 4: h_post_bda on the H_res / H_post the GPU stored
    gHr, gHp = h64(f["H_res"]), h64(f["H_post"])
    assert_act("out", out, O.h_post_bda_fwd(X64, gHr, gHp, x64, b64), w.act)

    # the chain end to end: out from the synthetic inputs alone.  First order, the errors of H_res
    # (Sinkhorn rule plus the logit tolerance carried through the map, as assert_h_res) and of
    # H_post (1e-5 relative) reach out[i] through sum_j dH_res[j][i] X[j] + dH_post[i] (x + bias),
    # on top of out's own rule.
    ro = O.h_post_bda_fwd(X64, ref["H_res"], ref["H_post"], x64, b64)
    tol_L = 1e-5 * (np.abs(ref["L"]) + np.sqrt(np.mean(ref["L"] ** 2)))
    bHr = 1e-5 * np.abs(ref["H_res"]) + 1.1 * h_res_chain_bound(ref["L"], w.iters, w.eps, tol_L)
    bHp = 1e-5 * np.abs(ref["H_post"])
    carried = np.einsum("tji,tjc->tic", bHr, np.abs(X64)) + bHp[:, :, None] * np.abs(x64 + b64)[:, None, :]
    e2e = 1e-5 * (np.abs(ro) + np.sqrt(np.mean(ro * ro))) + carried
    err = np.abs(h64(out) - ro)
    log(f"  end to end: max |out - oracle| / bound = {np.max(err / e2e):.3f}")
    _report("out (end to end)", h64(out), ro, e2e)

    # h_post_bda backward on the GPU's stored H_res / H_post
    odX, odHr, odHp, odx, odb = O.h_post_bda_bwd(G64, X64, gHr, gHp, x64, b64)
    assert_act("post dX", dXp, odX, w.act)
    assert_mixed("dH_res", dHr, odHr)
    assert_mixed("dH_post", dHp, odHp)
    assert_act("dx", dx, odx, w.act)
    assert_tokensum("dbias", dbias, odb, np.abs(odx).sum(axis=0), w.act, sum_depth("rows", N))

    # pre backward on the upstream gradients the GPU stored (dH_post, dH_res) and g; its residual
    # gradient accumulates onto the GPU's h_post_bda dX
    rb = O.pre_bwd(g64, h64(dHp), h64(dHr), X64, W64, None, None, w.rms_eps, w.iters, w.eps)
    assert_mixed("dH_pre", bw["dH_pre"], rb["dH_pre"])
    assert_mixed("dlogits", bw["dlogits"], rb["dL"])
    assert_act("dX (three terms)", bw["dX"], h64(dXp) + rb["dX"], w.act)
    aW, aa, ab = pre_bwd_abs_parts(g64, h64(dHp), h64(dHr), X64, W64, None, None, w.rms_eps, w.iters, w.eps)
    assert_tokensum("dW", bw["dW"], rb["dW"], aW, depth=sum_depth("proj", N, C, act=w.act))
    assert_tokensum("dalpha", bw["dalpha"], rb["dalpha"], aa, depth=sum_depth("param", N))
    assert_tokensum("dhbias", bw["dhbias"], rb["dhbias"], ab, depth=sum_depth("param", N))
