"""The whole mHC step captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every libmhc call only launches kernels on the caller's stream
(zero fills are kernels, no memset or copy nodes), so a captured step must
give the same bits as the same calls made eagerly.  Replays are interleaved
with eager work and synchronisations, with new inputs copied into the
captured buffers before each replay, and every replay is compared with an
eager run on the same inputs.  Workspaces and outputs come from the graph's
memory pool (the binding allocates with torch.empty during capture).
"""
import numpy as np
import pytest
import torch

from gpu_util import log
from mhc_hyper_connection_proj_amd import binding as B

pytestmark = pytest.mark.gpu


def _step(X, W, G, s, n_iters=20):
    f = B.mhc_pre_fwd(X, W, iters=n_iters)
    x = (f["agg"].float() * s.float()).to(torch.bfloat16)
    out = B.mhc_h_post_bda_fwd(X, f["H_res"], f["H_post"], x)
    _, dHr, dHp, dx, _ = B.mhc_h_post_bda_bwd(G, X, f["H_res"], f["H_post"], x, want_dX=False)
    g = (dx.float() * s.float()).to(torch.bfloat16)
    b = B.mhc_pre_bwd(g, dHp, dHr, X, W, f["saved"], f["H_pre"], f["H_post"], f["H_res_logits"], iters=n_iters,
                      post_G=G, post_H_res=f["H_res"])
    y = B.mhc_rmsnorm_fwd(f["agg"], None, 1e-6)
    dxn, dgam = B.mhc_rmsnorm_bwd(g, f["agg"], torch.ones_like(s, dtype=torch.float32), 1e-6)
    return dict(H_res=f["H_res"], agg=f["agg"], out=out, dX=b["dX"], dW=b["dW"], dalpha=b["dalpha"],
                dhbias=b["dhbias"], y=y, dxn=dxn, dgam=dgam)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("n,C", [(4, 1024), (2, 520)])
def test_step_graph_replays_match_eager(n, C):
    log(f"graph capture n={n} C={C}")
    N = 300
    torch.manual_seed(0)
    dev = "cuda"
    X = torch.empty(N, n, C, dtype=torch.bfloat16, device=dev)
    G = torch.empty_like(X)
    W = torch.empty(n * C, n * n + 2 * n, device=dev)
    s = (torch.rand(C, device=dev) + 0.5).to(torch.bfloat16)

    def fill(seed):
        gen = torch.Generator(device=dev).manual_seed(seed)
        X.copy_(torch.randn(N, n, C, device=dev, generator=gen).to(torch.bfloat16))
        G.copy_(torch.randn(N, n, C, device=dev, generator=gen).to(torch.bfloat16))
        W.copy_(torch.randn(n * C, n * n + 2 * n, device=dev, generator=gen) * 0.02)

    fill(1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(X, W, G, s)  # warm-up on a side stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = _step(X, W, G, s)
    torch.cuda.synchronize()
    for rep, seed in enumerate((2, 3, 2, 4)):
        fill(seed)
        torch.cuda.synchronize()
        eager = _step(X, W, G, s)
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=dev).sum()  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for k, v in eager.items():
            assert torch.equal(_bits(captured[k]), _bits(v)), f"replay {rep}: {k} differs from the eager step"
