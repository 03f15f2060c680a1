"""GPU parity of the RMSNorm step after h_aggregate (standalone and fused into
the pre pass) against the fp64 oracle.

Inputs are seeded synthetic arrays; oracle inputs never come from the GPU.
Sizes span one to several 8-channel groups per thread, ragged token blocks of
the dgamma reduction (16 tokens per workgroup) and C up to 16384.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_act, assert_normed, assert_tokensum, dev, h64, log, sum_depth
from mhc_hyper_connection_proj_amd import binding as B
from mhc_hyper_connection_proj_amd import synth

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(11)


def store(a64, act):
    return O.round_f64_to_bf16_bits(a64) if act == "bf16" else np.ascontiguousarray(a64, np.float32)


NORM_SHAPES = [("bf16", 1, 8), ("bf16", 37, 296), ("bf16", 33, 7168), ("f32", 17, 1032), ("f32", 64, 256),
               ("bf16", 3, 16384), ("f32", 5, 12288), ("bf16", 130, 4096)]


@pytest.mark.parametrize("act,N,C", NORM_SHAPES)
@pytest.mark.parametrize("with_gamma", [False, True])
@pytest.mark.parametrize("accumulate", [False, True])
def test_rmsnorm_fwd_bwd(act, N, C, with_gamma, accumulate):
    log(f"rmsnorm act={act} N={N} C={C} gamma={with_gamma} accumulate={accumulate}")
    x = store(RNG.standard_normal((N, C)) * 2.0, act)
    x64 = h64(x)
    if N > 2:
        x64[1] = 0.0  # an all-zero row (a padded token)
        x = store(x64, act)
    gamma = np.ascontiguousarray(RNG.uniform(0.5, 1.5, C), np.float32) if with_gamma else None
    dy = store(RNG.standard_normal((N, C)), act)
    din = store(RNG.standard_normal((N, C)), act)
    eps = 1e-6
    gd = dev(gamma) if gamma is not None else None
    y = B.mhc_rmsnorm_fwd(dev(x), gd, eps)
    dxd = dev(din) if accumulate else None
    dx, dg = B.mhc_rmsnorm_bwd(dev(dy), dev(x), gd, eps, dx=dxd, accumulate_dx=accumulate, want_dgamma=True)
    torch.cuda.synchronize()
    g64 = h64(gamma) if gamma is not None else np.ones(C)
    yo, r = O.rmsnorm_fwd(x64, g64 if with_gamma else None, eps)
    assert_act("y", y, yo, act)
    dxo, dgo = O.rmsnorm_bwd(h64(dy), x64, g64, eps)
    if accumulate:
        dxo = dxo + h64(din)
    assert_act("dx", dx, dxo, act)
    assert_tokensum("dgamma", dg, dgo, (np.abs(h64(dy) * r[:, None] * x64)).sum(0), depth=sum_depth("rows", N))
    if N > 2:  # zero row: y exactly 0, dx = r gamma dy (+ din) only
        assert np.all(h64(y)[1] == 0.0)


def test_rmsnorm_eps_and_constant_rows():
    # constant rows give +-1 (times gamma) up to eps; a large eps visibly shrinks the row
    N, C = 6, 520
    x64 = np.repeat(np.array([1.0, -2.0, 0.5, 3.0, -0.25, 8.0])[:, None], C, axis=1)
    x = store(x64, "f32")
    for eps in (0.0, 1e-6, 0.5):
        y = B.mhc_rmsnorm_fwd(dev(x), None, eps)
        torch.cuda.synchronize()
        assert_act("y", y, O.rmsnorm_fwd(x64, None, eps)[0], "f32")
    y = h64(B.mhc_rmsnorm_fwd(dev(x), None, 0.0))
    np.testing.assert_allclose(y, np.sign(x64), rtol=1e-6)


@pytest.mark.parametrize("act,N,C", [("bf16", 40, 7168), ("f32", 19, 256), ("bf16", 70, 1032)])
@pytest.mark.parametrize("with_gamma", [False, True])
def test_pre_rmsnorm_fwd(act, N, C, with_gamma):
    log(f"pre rmsnorm fwd act={act} N={N} C={C} gamma={with_gamma}")
    X = store(RNG.standard_normal((N, 4, C)), act)
    W = np.ascontiguousarray(RNG.standard_normal((4 * C, 24)) * 0.02, np.float32)
    gamma = np.ascontiguousarray(RNG.uniform(0.5, 1.5, C), np.float32) if with_gamma else None
    gd = dev(gamma) if gamma is not None else None
    f = B.mhc_pre_rmsnorm_fwd(dev(X), dev(W), gd, norm_eps=1e-6)
    p = B.mhc_pre_fwd(dev(X), dev(W))
    alone = B.mhc_rmsnorm_fwd(p["agg"], gd, 1e-6)
    torch.cuda.synchronize()
    # the fused pass equals the pre pass followed by the standalone norm, bit for bit
    for k in ("H_pre", "H_post", "H_res", "H_res_logits", "saved", "agg"):
        assert torch.equal(f[k], p[k]), k
    assert torch.equal(f["normed"].view(torch.int16 if act == "bf16" else torch.int32),
                       alone.view(torch.int16 if act == "bf16" else torch.int32))
    # against the oracle: agg (one rounding), then the norm of the oracle's stored agg, with the GPU's
    # measured agg deviation carried through the norm
    ref = O.pre_fwd(h64(X), h64(W))
    assert_act("agg", f["agg"], ref["agg"], act)
    assert_normed("normed", f["normed"], f["agg"], ref["agg"], h64(gamma) if gamma is not None else None, 1e-6, act)


def test_rmsnorm_zero_tokens_and_invalid():
    C = 64
    x = torch.zeros(0, C, dtype=torch.bfloat16, device="cuda")
    y = B.mhc_rmsnorm_fwd(x)
    dx, dg = B.mhc_rmsnorm_bwd(x, x, want_dgamma=True)
    torch.cuda.synchronize()
    assert y.shape == (0, C) and dx.shape == (0, C)
    assert torch.equal(dg, torch.zeros(C, device="cuda"))
    bad = torch.zeros(3, 12, dtype=torch.bfloat16, device="cuda")  # C % 8 != 0
    with pytest.raises(RuntimeError):
        B.mhc_rmsnorm_fwd(bad)
    xs = torch.zeros(3, 16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        B.mhc_rmsnorm_fwd(xs, eps=-1.0)


def test_rmsnorm_deterministic_bitwise():
    N, C = 300, 7168
    x = dev(store(RNG.standard_normal((N, C)), "bf16"))
    dy = dev(store(RNG.standard_normal((N, C)), "bf16"))
    gam = dev(np.ascontiguousarray(RNG.uniform(0.5, 1.5, C), np.float32))
    a = B.mhc_rmsnorm_bwd(dy, x, gam)
    b = B.mhc_rmsnorm_bwd(dy, x, gam)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("n,act,N,C", [(4, "bf16", 40, 7168), (4, "f32", 19, 256), (4, "bf16", 70, 1032),
                                       (2, "bf16", 37, 296), (8, "bf16", 21, 264)])
@pytest.mark.parametrize("gamma_on,fork_on,post", [(True, True, True), (False, False, False), (True, False, False),
                                                   (False, True, True)])
def test_pre_rmsnorm_bwd(n, act, N, C, gamma_on, fork_on, post):
    """mhc_pre_rmsnorm_bwd equals mhc_rmsnorm_bwd followed by mhc_pre_bwd bit for bit (the pre backward is
    held to the oracle on seeded inputs by the pre pass tests); its d_agg and dgamma against the oracle.
    Forward state, agg and H_res of the h_post_bda term come from the oracle (rounded to storage)."""
    log(f"pre rmsnorm bwd n={n} act={act} N={N} C={C} gamma={gamma_on} fork={fork_on} post={post}")
    J = n * n + 2 * n
    X = store(RNG.standard_normal((N, n, C)), act)
    W = np.ascontiguousarray(RNG.standard_normal((n * C, J)) * 0.02, np.float32)
    gamma = np.ascontiguousarray(RNG.uniform(0.5, 1.5, C), np.float32) if gamma_on else None
    gd = dev(gamma) if gamma is not None else None
    ref = O.pre_fwd(h64(X), h64(W), None, None, 1e-6, 20, 1e-6)
    f32 = lambda a: np.ascontiguousarray(a, np.float32)
    saved = np.zeros((N, B.saved_stride(n)), np.float32)
    saved[:, 0] = ref["r"]; saved[:, 1] = ref["q"]; saved[:, 2:2 + J] = ref["z"]
    agg = store(ref["agg"], act)
    dy = store(RNG.standard_normal((N, C)), act)
    fork = store(RNG.standard_normal((N, C)), act) if fork_on else None
    dHq = f32(RNG.standard_normal((N, n)))
    dHr = f32(RNG.standard_normal((N, n, n)))
    Gp = store(RNG.standard_normal((N, n, C)), act) if post else None
    Hrp = f32(O.sinkhorn_fwd(RNG.standard_normal((N, n, n)), 20, 1e-6)) if post else None
    kw = dict(post_G=dev(Gp), post_H_res=dev(Hrp)) if post else {}
    common = (dev(dHq), dev(dHr), dev(X), dev(W), dev(saved), dev(f32(ref["H_pre"])), dev(f32(ref["H_post"])),
              dev(f32(ref["L"])))
    fused = B.mhc_pre_rmsnorm_bwd(dev(dy), dev(agg), *common, gamma=gd, norm_eps=1e-6,
                                  g_fork=dev(fork) if fork_on else None, want_dgamma=True, want_d_agg=True, **kw)
    d_agg, dgam = B.mhc_rmsnorm_bwd(dev(dy), dev(agg), gd, 1e-6, dx=dev(fork).clone() if fork_on else None,
                                    accumulate_dx=fork_on, want_dgamma=True)
    pb = B.mhc_pre_bwd(d_agg, *common, **kw)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    assert torch.equal(bits(fused["d_agg"]), bits(d_agg)), "d_agg"
    assert torch.equal(bits(fused["dgamma"]), bits(dgam)), "dgamma"
    for k in ("dX", "dW", "dalpha", "dhbias"):
        assert torch.equal(bits(fused[k]), bits(pb[k])), k
    agg64 = h64(agg)
    odx, odg = O.rmsnorm_bwd(h64(dy), agg64, h64(gamma) if gamma_on else np.ones(C), 1e-6)
    assert_act("d_agg", fused["d_agg"], odx + (h64(fork) if fork_on else 0.0), act)
    r = O.rmsnorm_fwd(agg64, None, 1e-6)[1]
    assert_tokensum("dgamma", fused["dgamma"], odg, np.abs(h64(dy) * r[:, None] * agg64).sum(0),
                    depth=sum_depth("rows", N))
