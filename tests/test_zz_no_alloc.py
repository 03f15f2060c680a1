"""mhc_pre_fwd_noalloc (a static device scratch array, no workspace) against mhc_pre_fwd, through the C ABI.

Both forms run the same kernels, so every output must be bit-identical.  The calls come in a row on
one stream, larger then smaller inputs, so the static scratch holds the previous call's contents
when the next one starts; the workspace form gets a workspace filled with NaN bytes, so a kernel
that read scratch it had not written in the same call would show in either comparison.
"""
import numpy as np
import pytest
import torch

from mhc_hyper_connection_proj_amd import _lib as L

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _run(noalloc, X, W, alpha, hbias, n, iters=20):
    N, _, C = X.shape
    act = L.MHC_BF16 if X.dtype == torch.bfloat16 else L.MHC_F32
    dev = X.device
    nan = float("nan")
    o = {"H_pre": torch.full((N, n), nan, device=dev), "H_post": torch.full((N, n), nan, device=dev),
         "H_res": torch.full((N, n, n), nan, device=dev), "H_res_logits": torch.full((N, n, n), nan, device=dev),
         "saved": torch.full((N, L.lib().mhc_saved_stride(n)), nan, device=dev),
         "agg": torch.full((N, C), nan, dtype=X.dtype, device=dev)}
    ptr = lambda t: t.data_ptr() if t is not None else None
    args = [torch.cuda.current_stream().cuda_stream, N, n, C, act, X.data_ptr(), W.data_ptr(), ptr(alpha), ptr(hbias),
            1e-6, iters, 1e-6, *(o[k].data_ptr() for k in ("H_pre", "H_post", "H_res", "H_res_logits", "saved", "agg"))]
    lib = L.lib()
    if noalloc:
        L.check(lib.mhc_pre_fwd_noalloc(*args))
    else:
        wsb = lib.mhc_pre_fwd_workspace_size(N, n, C, act)
        ws = torch.full((max(wsb, 16),), 0xFF, dtype=torch.uint8, device=dev)  # NaN bytes
        L.check(lib.mhc_pre_fwd(*args, ws.data_ptr(), wsb))
    return o


# (n, act, tokens, C): the first call is the largest, each later one reads a scratch left by others
# (C = 4096 at n = 4 and C = 8192 at n = 2 take the staggered projection walk)
CASES = [(4, "bf16", 16384, 7168), (4, "bf16", 2000, 4096), (4, "bf16", 1000, 2048), (4, "bf16", 37, 296),
         (8, "bf16", 50, 296), (4, "f32", 20, 256), (2, "bf16", 3000, 8192), (2, "bf16", 3000, 1024),
         (4, "bf16", 5, 8)]


def test_noalloc_pre_fwd_matches_workspace_form():
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(11)
    for n, act, N, C in CASES:
        print(f"noalloc pre fwd n={n} act={act} N={N} C={C}", flush=True)
        dt = torch.bfloat16 if act == "bf16" else torch.float32
        J = n * n + 2 * n
        X = torch.randn(N, n, C, device=dev, generator=gen).to(dt)
        W = torch.randn(n * C, J, device=dev, generator=gen) * 0.02
        alpha = torch.tensor([1.3, 0.7, 1.1], device=dev)
        hbias = torch.randn(J, device=dev, generator=gen) * 0.1
        a = _run(True, X, W, alpha, hbias, n)
        b = _run(False, X, W, alpha, hbias, n)
        torch.cuda.synchronize()
        for k in a:
            assert not torch.isnan(a[k].float()).any(), f"{k}: not fully written"
            assert torch.equal(_bits(a[k]), _bits(b[k])), f"n={n} {act} N={N} C={C}: {k} differs"


def test_noalloc_pre_fwd_rejects_beyond_scratch_on_gpu():
    """Past the static scratch the call fails before enqueueing: its outputs keep their contents."""
    dev = torch.device("cuda", 0)
    N, n, C = 300000, 4, 8
    X = torch.zeros(N, n, C, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(n * C, 24, device=dev)
    outs = [torch.full(s, 7.0, device=dev) for s in ((N, 4), (N, 4), (N, 4, 4), (N, 4, 4))]
    agg = torch.full((N, C), 7.0, dtype=torch.bfloat16, device=dev)
    st = L.lib().mhc_pre_fwd_noalloc(torch.cuda.current_stream().cuda_stream, N, n, C, L.MHC_BF16, X.data_ptr(),
                                     W.data_ptr(), None, None, 1e-6, 20, 1e-6, *(t.data_ptr() for t in outs), None,
                                     agg.data_ptr())
    torch.cuda.synchronize()
    assert st == L.STATUS.index("MHC_ERR_UNSUPPORTED")
    assert all(bool((t == 7.0).all()) for t in outs) and bool((agg == 7.0).all())
