"""CPU tests of the C ABI boundary: symbols, status strings, fail-closed validation.

No kernel is launched: every call here fails validation on the host, before
any HIP runtime call, so the pointers are plain integers that are never
dereferenced.
"""
import ctypes
import os
import subprocess

import pytest
import torch

from mhc_hyper_connection_proj_amd import _lib as L

# The fake pointers below must never reach a kernel: with a GPU visible, a call
# that slipped through validation would launch on invalid addresses.
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="host-only validation tests use fake device pointers")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WS, ARG = range(8)
A = 0x7f0000000000  # fake, 16-byte aligned device addresses, far apart
MB = 1 << 20


def p(i):
    return A + i * 64 * MB


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from mhc_hyper_connection_proj_amd import build
        build.build()
    return L.lib()


def test_exports_every_header_symbol(lib):
    declared = L.header_functions()
    assert len(declared) >= 18
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for f in declared:
        assert hasattr(lib, f)
    assert set(declared) == set(L.SIGNATURES)


def test_status_strings_and_version(lib):
    for i, name in enumerate(L.STATUS):
        assert lib.mhc_status_string(i).decode() == name
    assert b"gfx950" in lib.mhc_version()


def _last(lib):
    return lib.mhc_last_error().decode()


def test_variant_entry_points_validate_before_launch(lib):
    E = {n: i for i, n in enumerate(L.STATUS)}
    fake = 0x10000
    # n > 8, C % 8 != 0, NULL inputs, a misaligned output: all rejected on the host
    assert lib.mhc_stream_mix_fwd(None, 4, 9, 64, 0, fake, fake + 8192, fake + 16384) == E["MHC_ERR_UNSUPPORTED"]
    assert lib.mhc_stream_mix_fwd(None, 4, 4, 60, 0, fake, fake + 4096, fake + 8192) == E["MHC_ERR_UNSUPPORTED"]
    assert lib.mhc_stream_mix_bwd(None, 4, 4, 64, 0, None, fake, fake, fake, fake) == E["MHC_ERR_NULL"]
    assert lib.mhc_stream_distribute_fwd(None, 4, 4, 64, 0, fake, fake + 4096, fake + 8200) == E["MHC_ERR_ALIGN"]
    assert lib.mhc_stream_distribute_bwd(None, 4, 4, 64, 0, fake, None, fake, fake, fake) == E["MHC_ERR_NULL"]
    assert lib.mhc_h_aggregate_static_fwd(None, 4, 4, 64, 0, fake, None, fake + 8192) == E["MHC_ERR_NULL"]
    # the shared-row backward needs a workspace of 16 bytes per token
    assert lib.mhc_h_aggregate_static_bwd_workspace_size(100, 4, 64, 0) == 1600
    st = lib.mhc_h_aggregate_static_bwd(None, 100, 4, 64, 0, fake, fake + (1 << 20), fake + (2 << 20),
                                        fake + (3 << 20), 0, fake + (4 << 20), fake + (5 << 20), 16)
    assert st == E["MHC_ERR_WORKSPACE"]
    # overlapping output and input
    assert lib.mhc_stream_mix_fwd(None, 4, 4, 64, 0, fake, fake + 8192, fake + 1024) == E["MHC_ERR_ALIAS"]


def test_kernel_events_hook_validation(lib):
    # handles are only stored (no HIP call is made until a kernel launches)
    fake = 0x1000
    assert lib.mhc_set_kernel_events(L.MHC_KERNEL_PROJ_BWD_DXDW, fake, fake + 64) == 0
    assert lib.mhc_set_kernel_events(7, fake, fake + 64) == L.STATUS.index("MHC_ERR_ARG")
    assert "unknown kernel id" in _last(lib)
    assert lib.mhc_set_kernel_events(L.MHC_KERNEL_PROJ_BWD_DXDW, fake, None) == L.STATUS.index("MHC_ERR_ARG")
    assert lib.mhc_set_kernel_events(L.MHC_KERNEL_PROJ_BWD_DXDW, None, None) == 0  # clears
    assert lib.mhc_set_kernel_events(L.MHC_KERNEL_NONE, fake, fake) == 0  # clears


def test_sinkhorn_validation(lib):
    f = lib.mhc_sinkhorn_fwd
    assert f(None, -1, 4, p(0), p(1), 20, 1e-6) == SHAPE
    assert f(None, 10, 9, p(0), p(1), 20, 1e-6) == UNSUP
    assert f(None, 10, 0, p(0), p(1), 20, 1e-6) == SHAPE
    assert f(None, 10, 4, p(0), p(1), -1, 1e-6) == ARG
    assert f(None, 10, 4, p(0), p(1), 5000, 1e-6) == UNSUP
    assert f(None, 10, 4, p(0), p(1), 20, -1e-6) == ARG
    assert f(None, 10, 4, p(0), p(1), 20, float("nan")) == ARG
    assert f(None, 10, 4, None, p(1), 20, 1e-6) == NULL and "logits" in _last(lib)
    assert f(None, 10, 4, p(0) + 4, p(1), 20, 1e-6) == ALIGN
    assert f(None, 10, 4, p(0), p(0) + 320, 20, 1e-6) == ALIAS   # 10*64 bytes: overlaps
    assert f(None, 0, 4, None, None, 20, 1e-6) == OK              # empty: no-op
    g = lib.mhc_sinkhorn_bwd
    assert g(None, 10, 4, p(0), p(1), p(1), 20, 1e-6) == ALIAS
    assert g(None, 10, 4, p(0), None, p(2), 20, 1e-6) == NULL


def test_dims_validation(lib):
    f = lib.mhc_h_aggregate_fwd
    assert f(None, 4, 4, 63, 0, p(0), p(1), p(2)) == UNSUP       # C % 8
    assert f(None, 4, 4, 0, 0, p(0), p(1), p(2)) == SHAPE
    assert f(None, 4, 4, 16392, 0, p(0), p(1), p(2)) == UNSUP    # C > 16384
    assert f(None, 4, 9, 64, 0, p(0), p(1), p(2)) == UNSUP       # n > 8
    assert f(None, 4, 0, 64, 0, p(0), p(1), p(2)) == SHAPE       # n < 1
    assert f(None, 4, 4, 64, 7, p(0), p(1), p(2)) == ARG         # dtype
    assert f(None, -2, 4, 64, 0, p(0), p(1), p(2)) == SHAPE
    assert f(None, 0, 4, 64, 0, None, None, None) == OK
    assert f(None, 4, 4, 64, 0, p(0), p(1), p(0) + 1024) == ALIAS  # out inside X (4*4*64*2 bytes)


def test_post_bwd_validation(lib):
    f = lib.mhc_h_post_bda_bwd
    # stream, tokens, n, C, act, G, X, H_res, H_post, x, bias, dX, dH_res, dH_post, dx, dbias, ws, ws_bytes
    args = [None, 8, 4, 64, 0, p(0), p(1), p(2), p(3), p(4), None, p(5), p(6), p(7), p(8), None, None, 0]
    # dbias without bias
    a = list(args); a[15] = p(9)
    assert f(*a) == ARG
    # dbias with bias but no workspace
    a = list(args); a[10] = p(10); a[15] = p(9)
    assert f(*a) == WS
    need = lib.mhc_h_post_bda_bwd_workspace_size(8, 4, 64, 0, 1)
    assert need > 0
    a[16] = p(11); a[17] = need - 1
    assert f(*a) == WS
    a[17] = need; a[16] = p(11) + 8
    assert f(*a) == ALIGN
    # outputs overlapping each other
    a = list(args); a[12] = p(5)
    assert f(*a) == ALIAS
    assert lib.mhc_h_post_bda_bwd_workspace_size(8, 4, 64, 0, 0) == 0


def test_proj_validation(lib):
    f = lib.mhc_proj_rms_h
    need = lib.mhc_proj_rms_h_workspace_size(70, 4, 4096, 0)
    assert need > 0
    base = [None, 70, 4, 4096, 0, p(0), p(1), None, None, 1e-6, p(2), p(3), p(4), p(5), p(6), need]
    a = list(base); a[9] = -1.0
    assert f(*a) == ARG
    a = list(base); a[14] = None
    assert f(*a) == WS
    a = list(base); a[6] = None
    assert f(*a) == NULL
    a = list(base); a[12] = p(0) + 4096
    assert f(*a) == ALIAS
    a = list(base); a[13] = p(6)                                  # saved == workspace
    assert f(*a) == ALIAS
    g = lib.mhc_proj_rms_h_bwd
    nb = lib.mhc_proj_rms_h_bwd_workspace_size(70, 4, 4096, 0)
    b = [None, 70, 4, 4096, 0, p(0), p(1), None, p(2), p(3), p(4), p(5), p(6), p(7), p(0), 1, p(9), None, None,
         p(10), nb]
    assert g(*b) == ALIAS                                          # dX aliases X
    b[14] = p(8)
    b[19] = None
    assert g(*b) == WS
    assert g(None, 0, 4, 64, 0, None, None, None, None, None, None, None, None, None, None, 0, None, None, None,
             None, 0) == OK


def test_pre_validation(lib):
    f = lib.mhc_pre_fwd
    ws = lib.mhc_pre_fwd_workspace_size(16, 4, 256, 1)
    base = [None, 16, 4, 256, 1, p(0), p(1), None, None, 1e-6, 20, 1e-6, p(2), p(3), p(4), p(5), None, p(6),
            p(7), ws]
    a = list(base); a[10] = -3
    assert f(*a) == ARG
    a = list(base); a[11] = float("inf")
    assert f(*a) == ARG
    a = list(base); a[17] = p(4)
    assert f(*a) == ALIAS
    g = lib.mhc_pre_bwd
    wb = lib.mhc_pre_bwd_workspace_size(16, 4, 256, 1)
    b = [None, 16, 4, 256, 1, p(0), p(1), p(2), p(3), p(4), None, p(5), p(6), p(7), p(8), 20, 1e-6, None, None,
         p(9), 1, p(10), None, None, None, None, p(11), wb]
    b2 = list(b); b2[5] = None
    assert g(*b2) == NULL
    b2 = list(b); b2[19] = p(3)                                    # dX aliases X
    assert g(*b2) == ALIAS
    b2 = list(b); b2[27] = wb - 16
    assert g(*b2) == WS
    b2 = list(b); b2[17] = p(12)                                   # post_G without post_H_res
    assert g(*b2) == ARG
    b2 = list(b); b2[17] = p(12); b2[18] = p(13); b2[19] = p(12)   # dX aliases post_G
    assert g(*b2) == ALIAS


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        L.lib()


def test_general_n_sizes(lib):
    # saved-state stride and workspace queries for every supported n
    assert [lib.mhc_saved_stride(n) for n in range(0, 10)] == [0, 32, 32, 32, 32, 40, 56, 72, 88, 0]
    for n in (1, 2, 3, 5, 8):
        assert lib.mhc_proj_rms_h_workspace_size(100, n, 64, 0) > 0
        assert lib.mhc_proj_rms_h_bwd_workspace_size(100, n, 64, 0) > 0
        assert lib.mhc_h_aggregate_static_bwd_workspace_size(100, n, 64, 0) == 100 * n * 4
    assert lib.mhc_proj_rms_h_workspace_size(100, 9, 64, 0) == 0
    # buffer sizes follow n: X of 4 tokens x 8 streams x 64 bf16 = 4096 bytes, so an output 4000 bytes in overlaps
    f = lib.mhc_h_aggregate_fwd
    assert f(None, 4, 8, 64, 0, p(0), p(1), p(0) + 4000) == ALIAS
    assert f(None, 4, 2, 64, 0, p(0), p(1), p(0) + 1008) == ALIAS  # X: 4 x 2 x 64 bf16 = 1024 bytes


def test_rmsnorm_validation(lib):
    # every call below must fail validation: the pointers are fake
    f = lib.mhc_rmsnorm_fwd
    # stream, tokens, C, act, x, gamma, eps, y
    assert f(None, 4, 60, 0, p(0), None, 1e-6, p(1)) == UNSUP                 # C % 8
    assert f(None, 4, 64, 0, p(0), None, -1.0, p(1)) == ARG                   # eps < 0
    assert f(None, 4, 64, 0, None, None, 1e-6, p(1)) == NULL and "x" in _last(lib)
    assert f(None, 4, 64, 0, p(0), None, 1e-6, p(0) + 256) == ALIAS           # y inside x (4*64*2 bytes)
    assert f(None, 4, 64, 0, p(0), p(0) + 64, 1e-6, p(0) + 128) == ALIAS      # y inside x, gamma given
    assert f(None, 0, 64, 0, None, None, 1e-6, None) == OK                    # empty: no-op
    g = lib.mhc_rmsnorm_bwd
    # stream, tokens, C, act, dy, x, gamma, eps, dx, accumulate, dgamma, ws, ws_bytes
    need = lib.mhc_rmsnorm_bwd_workspace_size(100, 64, 0, 1)
    assert need >= (7 + 16) * 64 * 4 and lib.mhc_rmsnorm_bwd_workspace_size(100, 64, 0, 0) == 0
    assert g(None, 100, 64, 0, p(0), p(1), None, 1e-6, p(2), 0, p(3), None, 0) == WS
    assert g(None, 100, 64, 0, p(0), p(1), None, 1e-6, p(0), 0, None, None, 0) == ALIAS   # dx is dy
    assert g(None, 100, 64, 0, p(0), None, None, 1e-6, p(2), 0, None, None, 0) == NULL
    h = lib.mhc_pre_rmsnorm_fwd
    # stream, tokens, n, C, act, X, W, alpha, hbias, rms_eps, iters, eps, gamma, norm_eps,
    # H_pre, H_post, H_res, logits, saved, agg, normed, ws, ws_bytes
    ws = lib.mhc_pre_fwd_workspace_size(8, 4, 64, 0)
    assert h(None, 8, 4, 64, 0, p(0), p(1), None, None, 1e-6, 20, 1e-6, None, 1e-6,
             p(2), p(3), p(4), p(5), None, p(6), p(6) + 64, p(7), ws) == ALIAS     # normed inside agg
    assert h(None, 8, 4, 64, 0, p(0), p(1), None, None, 1e-6, 20, 1e-6, None, -1.0,
             p(2), p(3), p(4), p(5), None, p(6), p(8), p(7), ws) == ARG            # norm_eps < 0


def test_token_count_limit_rejected_before_launch(lib):
    """tokens (or a Sinkhorn count) above 2^22 would take some launch past 2^31 threads: rejected on the
    host with MHC_ERR_UNSUPPORTED, before anything is enqueued; 2^22 itself passes the check and stops
    at the next one (a missing input)."""
    E = {n: i for i, n in enumerate(L.STATUS)}
    big = (1 << 22) + 1
    fake = 0x10000
    assert lib.mhc_h_aggregate_fwd(None, big, 1, 8, 0, fake, fake, fake) == E["MHC_ERR_UNSUPPORTED"]
    assert "4194304" in _last(lib)
    assert lib.mhc_rmsnorm_fwd(None, big, 8, 0, fake, None, 1e-6, fake) == E["MHC_ERR_UNSUPPORTED"]
    assert lib.mhc_sinkhorn_fwd(None, big, 4, fake, fake, 20, 1e-6) == E["MHC_ERR_UNSUPPORTED"]
    assert lib.mhc_sinkhorn_bwd(None, big, 2, fake, fake, fake, 20, 1e-6) == E["MHC_ERR_UNSUPPORTED"]
    assert lib.mhc_pre_fwd(None, big, 4, 8, 0, fake, fake, None, None, 1e-6, 20, 1e-6, fake, fake, fake, fake,
                           None, fake, fake, 1 << 30) == E["MHC_ERR_UNSUPPORTED"]
    for q in (lib.mhc_pre_fwd_workspace_size, lib.mhc_pre_bwd_workspace_size, lib.mhc_proj_rms_h_workspace_size):
        assert q(big, 4, 8, 0) == 0 and q(1 << 22, 4, 8, 0) > 0
    # at the limit the token check passes and the missing X is reported instead
    assert lib.mhc_h_aggregate_fwd(None, 1 << 22, 1, 8, 0, None, fake, fake) == E["MHC_ERR_NULL"]


def test_noalloc_pre_fwd_rejects_beyond_its_scratch(lib):
    """mhc_pre_fwd_noalloc: a call whose scratch need exceeds the static array is rejected on the host,
    before any HIP call (300000 tokens at n = 4, C = 8 need 8 split-K rows of 128 bytes per token)."""
    E = {n: i for i, n in enumerate(L.STATUS)}
    N = 300000
    assert lib.mhc_pre_fwd_workspace_size(N, 4, 8, 0) > 64 << 20
    st = lib.mhc_pre_fwd_noalloc(None, N, 4, 8, 0, p(0), p(1), None, None, 1e-6, 20, 1e-6, p(2), p(3), p(4), p(5),
                                 None, p(6))
    assert st == E["MHC_ERR_UNSUPPORTED"]
    assert "static scratch" in _last(lib)
    # the same checks as mhc_pre_fwd come first
    assert lib.mhc_pre_fwd_noalloc(None, 4, 4, 8, 0, None, p(1), None, None, 1e-6, 20, 1e-6, p(2), p(3), p(4), p(5),
                                   None, p(6)) == E["MHC_ERR_NULL"]
    assert lib.mhc_pre_fwd_noalloc(None, 4, 4, 8, 0, p(0), p(1), None, None, 1e-6, -1, 1e-6, p(2), p(3), p(4), p(5),
                                   None, p(6)) == E["MHC_ERR_ARG"]
    assert lib.mhc_pre_fwd_noalloc(None, 0, 4, 8, 0, None, None, None, None, 1e-6, 20, 1e-6, None, None, None, None,
                                   None, None) == E["MHC_OK"]
