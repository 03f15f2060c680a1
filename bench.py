"""Benchmark of the per-token mHC path on one MI355X.

Default workload (one GPU): B=4, T=4096 (16384 tokens), n=4, C=7168, bf16
residual; the layer between h_aggregate and h_post_bda is a fixed per-channel
bf16 scale.  One step = pre pass forward (projection + RMS + compute_h +
Sinkhorn + h_aggregate) -> layer -> h_post_bda forward -> h_post_bda backward
-> layer backward -> pre pass backward (accumulated onto the h_post_bda dX).

Timing: W untimed warmup steps, then K timed steps between synchronisations.
HIP events on the launch stream bracket every phase; the mHC time of a step
is the sum of its four mHC phases (the layer stand-in is not part of the
path and is reported separately).  value = tokens / mHC time.

Prints one JSON line.  `--gpus N` with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "tokens/s and achieved HBM GB/s (% of peak), mHC pre+post fwd+bwd, n=4"


def ledger_bytes_per_token(C: int, N: int) -> dict:
    """Algorithmic HBM bytes per token: every boundary tensor read or written once per phase."""
    K = 4 * C
    w_amort = K * 24 * 4 / N  # W read (fwd), W read + dW write (bwd), amortised over the tokens
    phases = {
        "pre_fwd": 8 * C + 2 * C + 16 + 16 + 64 + 64 + 128 + w_amort,
        "post_fwd": 8 * C + 2 * C + 64 + 16 + 8 * C,
        # the post backward's dX term is formed inside the pre backward from G
        # (read there instead of a materialised dX), so dX is written once
        "post_bwd": 8 * C + 8 * C + 2 * C + 64 + 16 + 2 * C + 64 + 16,
        "pre_bwd": 2 * C + 8 * C + 8 * C + 64 + 16 + 64 + 128 + 16 + 16 + 64 + 8 * C + 2 * w_amort,
    }
    phases["total"] = sum(phases.values())
    # the dX / dW kernel of the pre backward (the dominant kernel): X, g and
    # the h_post_bda upstream gradient G in, dX out, H_pre and H_res rows
    phases["dxdw_kernel"] = 8 * C + 2 * C + 8 * C + 8 * C + 16 + 64
    return phases


def src_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def pmc_traffic(name: str, sources) -> float | None:
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    reported only while the kernel's sources are the ones that were measured."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = dict(line.split(" = ", 1) for line in open(path).read().splitlines()
               if " = " in line and not line.startswith("#"))
    if rec.get("src_hash") != src_hash(sources):
        return None
    return float(rec["hbm_bytes_per_launch"])


def measure_variants(lib, L, sp, N, n, C, X, G, H_res, H_post, x, g, out, dX, dM, dH, dx, stream, torch):
    """The h_post_bda halves and the shared-row h_aggregate at the same size, after the timed
    steps: mean of 5 event-timed calls each; GB/s on algorithmic bytes (each tensor once)."""
    from mhc_hyper_connection_proj_amd._lib import MHC_BF16
    P = lambda t: t.data_ptr()
    dev = X.device
    h = torch.tensor([0.4, 0.3, 0.2, 0.1], device=dev)
    dh = torch.empty(4, device=dev)
    wsn = lib.mhc_h_aggregate_static_bwd_workspace_size(N, n, C, MHC_BF16)
    ws = torch.empty(max(wsn, 16), dtype=torch.uint8, device=dev)
    calls = {
        "stream_mix_fwd": (16 * C + 64, lambda: lib.mhc_stream_mix_fwd(sp, N, n, C, MHC_BF16, P(X), P(H_res), P(out))),
        "stream_mix_bwd": (24 * C + 128, lambda: lib.mhc_stream_mix_bwd(sp, N, n, C, MHC_BF16, P(G), P(X), P(H_res),
                                                                         P(dX), P(dM))),
        "stream_distribute_fwd": (10 * C + 16, lambda: lib.mhc_stream_distribute_fwd(sp, N, n, C, MHC_BF16, P(x),
                                                                                      P(H_post), P(out))),
        "stream_distribute_bwd": (12 * C + 32, lambda: lib.mhc_stream_distribute_bwd(sp, N, n, C, MHC_BF16, P(G), P(x),
                                                                                      P(H_post), P(dx), P(dH))),
        "h_aggregate_static_fwd": (10 * C, lambda: lib.mhc_h_aggregate_static_fwd(sp, N, n, C, MHC_BF16, P(X), P(h),
                                                                                   P(x))),
        "h_aggregate_static_bwd": (18 * C, lambda: lib.mhc_h_aggregate_static_bwd(sp, N, n, C, MHC_BF16, P(g), P(X),
                                                                                   P(h), P(dX), 0, P(dh), P(ws), wsn)),
    }
    # RMSNorm of the aggregated stream [N][C] (x as its input, g as its upstream gradient), with a gain
    gam = torch.linspace(0.5, 1.5, C, device=dev)
    dgam = torch.empty(C, device=dev)
    wsr = lib.mhc_rmsnorm_bwd_workspace_size(N, C, MHC_BF16, 1)
    wsn_ = torch.empty(max(wsr, 16), dtype=torch.uint8, device=dev)
    calls["rmsnorm_fwd"] = (4 * C, lambda: lib.mhc_rmsnorm_fwd(sp, N, C, MHC_BF16, P(x), P(gam), 1e-6, P(dx)))
    calls["rmsnorm_bwd"] = (6 * C, lambda: lib.mhc_rmsnorm_bwd(sp, N, C, MHC_BF16, P(g), P(x), P(gam), 1e-6, P(dx), 0,
                                                                P(dgam), P(wsn_), wsr))
    # h_post_bda backward with a bias (dbias summed over tokens), dX left to the pre backward
    bias = torch.full((C,), 0.1, dtype=torch.bfloat16, device=dev)
    dbias = torch.empty(C, dtype=torch.bfloat16, device=dev)
    wsb = lib.mhc_h_post_bda_bwd_workspace_size(N, n, C, MHC_BF16, 1)
    wsb_ = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    calls["h_post_bda_bwd_dbias"] = (20 * C + 160, lambda: lib.mhc_h_post_bda_bwd(
        sp, N, n, C, MHC_BF16, P(G), P(X), P(H_res), P(H_post), P(x), P(bias), None, P(dM), P(dH), P(dx),
        P(dbias), P(wsb_), wsb))
    res = {}
    for name, (bytes_per_token, fn) in calls.items():
        L.check(fn())
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        evs[0].record(stream)
        for i in range(5):
            L.check(fn())
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([evs[i].elapsed_time(evs[i + 1]) for i in range(5)]))
        gbs = bytes_per_token * N / (ms * 1e-3) / 1e9
        res[name] = {"ms": ms, "algorithmic_bytes_per_token": bytes_per_token, "achieved_gbs": gbs,
                     "frac": gbs / HBM_PEAK_GBS}
    return res


def measure_projection_choice(lib, L, sp, stream, torch, X, W, N, n, C) -> dict:
    """The forward projection at the workload's shape with x @ W on the matrix cores (mhc_proj_rms_h)
    and as fp32 FMAs on the vector ALUs (mhc_proj_rms_h_fma), same inputs: mean of 5 event-timed calls
    each after one warm-up; GB/s on the residual read (8C bytes per token)."""
    dev = X.device
    e = lambda *sh: torch.empty(*sh, dtype=torch.float32, device=dev)
    Hp, Hq, Lg, sv = e(N, 4), e(N, 4), e(N, 4, 4), e(N, 32)
    wsb = lib.mhc_proj_rms_h_workspace_size(N, n, C, L.MHC_BF16)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    P = lambda t: t.data_ptr()
    res = {}
    for name, fn in (("mfma", lib.mhc_proj_rms_h), ("fma", lib.mhc_proj_rms_h_fma)):
        call = lambda: L.check(fn(sp, N, n, C, L.MHC_BF16, P(X), P(W), None, None, 1e-6, P(Hp), P(Hq), P(Lg), P(sv),
                                  P(ws), wsb))
        call()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record(stream)
        for i in range(5):
            call()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(5)]))
        res[name + "_ms"] = ms
        res[name + "_gbs"] = 8 * C * N / (ms * 1e-3) / 1e9
    return res


def measure_norm_bwd_fusion(lib, L, sp, stream, torch, N, n, C, X, W, G, H_res, agg, dy, saved, H_pre, H_post,
                            logits, dHp, dHr) -> dict:
    """The pre backward with the norm's backward in front, at the workload's shape (the h_post_bda term
    formed from G), with a gain and dgamma and without: mhc_pre_rmsnorm_bwd against mhc_rmsnorm_bwd
    followed by mhc_pre_bwd (the same results, bit for bit).  Mean of 5 event-timed calls of each
    after one warm-up, the two forms alternating."""
    dev = X.device
    bf = torch.bfloat16
    P = lambda t: t.data_ptr() if t is not None else None
    gam = torch.linspace(0.5, 1.5, C, device=dev)
    dgam = torch.empty(C, device=dev)
    dX = torch.empty(N, n, C, dtype=bf, device=dev)
    dagg = torch.empty(N, C, dtype=bf, device=dev)
    dW, da, db = (torch.empty(*sh, device=dev) for sh in ((n * C, 24), (3,), (24,)))
    wf = lib.mhc_pre_rmsnorm_bwd_workspace_size(N, n, C, L.MHC_BF16, 1)
    wsf = torch.empty(wf, dtype=torch.uint8, device=dev)
    wn = lib.mhc_rmsnorm_bwd_workspace_size(N, C, L.MHC_BF16, 1)
    wsn = torch.empty(wn, dtype=torch.uint8, device=dev)
    wp = lib.mhc_pre_bwd_workspace_size(N, n, C, L.MHC_BF16)
    wsp = torch.empty(wp, dtype=torch.uint8, device=dev)

    def fused():
        L.check(lib.mhc_pre_rmsnorm_bwd(sp, N, n, C, L.MHC_BF16, P(dy), P(agg), P(gam), 1e-6, None, P(dHp), P(dHr),
                                        P(X), P(W), None, P(saved), P(H_pre), P(H_post), P(logits), 20, 1e-6, P(G),
                                        P(H_res), P(dX), 0, P(dW), P(da), P(db), P(dgam), None, P(wsf), wf))

    def composed():
        L.check(lib.mhc_rmsnorm_bwd(sp, N, C, L.MHC_BF16, P(dy), P(agg), P(gam), 1e-6, P(dagg), 0, P(dgam), P(wsn), wn))
        L.check(lib.mhc_pre_bwd(sp, N, n, C, L.MHC_BF16, P(dagg), P(dHp), P(dHr), P(X), P(W), None, P(saved),
                                P(H_pre), P(H_post), P(logits), 20, 1e-6, P(G), P(H_res), P(dX), 0, P(dW), P(da),
                                P(db), None, None, P(wsp), wp))

    def fused_nog():
        L.check(lib.mhc_pre_rmsnorm_bwd(sp, N, n, C, L.MHC_BF16, P(dy), P(agg), None, 1e-6, None, P(dHp), P(dHr),
                                        P(X), P(W), None, P(saved), P(H_pre), P(H_post), P(logits), 20, 1e-6, P(G),
                                        P(H_res), P(dX), 0, P(dW), P(da), P(db), None, None, P(wsf), wf))

    def composed_nog():
        L.check(lib.mhc_rmsnorm_bwd(sp, N, C, L.MHC_BF16, P(dy), P(agg), None, 1e-6, P(dagg), 0, None, None, 0))
        L.check(lib.mhc_pre_bwd(sp, N, n, C, L.MHC_BF16, P(dagg), P(dHp), P(dHr), P(X), P(W), None, P(saved),
                                P(H_pre), P(H_post), P(logits), 20, 1e-6, P(G), P(H_res), P(dX), 0, P(dW), P(da),
                                P(db), None, None, P(wsp), wp))

    # the two forms alternate call by call (back-to-back calls of this phase slow down as the GPU
    # warms, which would otherwise favour whichever form runs first)
    res = {}
    for (na, fa), (nb, fb) in ((("fused_ms", fused), ("norm_then_pre_bwd_ms", composed)),
                               (("fused_no_gain_ms", fused_nog), ("norm_then_pre_bwd_no_gain_ms", composed_nog))):
        fa(); fb()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(11)]
        ev[0].record(stream)
        for i in range(5):
            fa()
            ev[2 * i + 1].record(stream)
            fb()
            ev[2 * i + 2].record(stream)
        torch.cuda.synchronize()
        res[na] = float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(5)]))
        res[nb] = float(np.mean([ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(5)]))
    return res


def measure_reread_chunks(lib, L, sp, stream, torch, Xcopies, W, G, bufs, N, n, C, rms_eps, iters, eps) -> dict:
    """The pre forward and the pre backward read X twice (the projection then the aggregate; the
    dH_pre pass then dX/dW).  Run on token chunks small enough for the 256 MB Infinity Cache, the
    second read of a chunk's X (and g) can come from there: each pass is called once per chunk
    (pointers offset into the same tensors; dW, dalpha, dhbias overwritten per chunk, which does
    not change the work), against one call over all tokens.  Mean of 4 event-timed passes after one
    warm-up, the two residual copies alternated between passes."""
    from mhc_hyper_connection_proj_amd._lib import MHC_BF16
    P = lambda t: t.data_ptr()
    b = bufs
    ws_f = lib.mhc_pre_fwd_workspace_size(N, n, C, MHC_BF16)
    ws_b = lib.mhc_pre_bwd_workspace_size(N, n, C, MHC_BF16)
    dev = G.device
    wsf = torch.empty(max(ws_f, 16), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(ws_b, 16), dtype=torch.uint8, device=dev)
    xs, hs = n * C * 2, C * 2  # bytes per token: residual rows, one row

    def fwd(X, t0, m):
        L.check(lib.mhc_pre_fwd(sp, m, n, C, MHC_BF16, P(X) + t0 * xs, P(W), None, None, rms_eps, iters, eps,
                                P(b["H_pre"]) + t0 * 16, P(b["H_post"]) + t0 * 16, P(b["H_res"]) + t0 * 64,
                                P(b["L"]) + t0 * 64, P(b["saved"]) + t0 * 128, P(b["agg"]) + t0 * hs, P(wsf), ws_f))

    def bwd(X, t0, m):
        L.check(lib.mhc_pre_bwd(sp, m, n, C, MHC_BF16, P(b["g"]) + t0 * hs, P(b["dHp"]) + t0 * 16,
                                P(b["dHr"]) + t0 * 64, P(X) + t0 * xs, P(W), None, P(b["saved"]) + t0 * 128,
                                P(b["H_pre"]) + t0 * 16, P(b["H_post"]) + t0 * 16, P(b["L"]) + t0 * 64, iters, eps,
                                P(G) + t0 * xs, P(b["H_res"]) + t0 * 64, P(b["dX"]) + t0 * xs, 0, P(b["dW"]),
                                P(b["da"]), P(b["db"]), None, None, P(wsb), ws_b))

    def timed(fn, chunk, reps=4):
        def one(k):
            X = Xcopies[k % 2]
            for t0 in range(0, N, chunk):
                fn(X, t0, min(chunk, N - t0))
        one(1)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for k in range(reps):
            one(k)
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[k].elapsed_time(ev[k + 1]) for k in range(reps)]))

    chunks = [N, 4096, 2048, 1024]
    return {"chunk_tokens": chunks, "pre_fwd_ms": [timed(fwd, c) for c in chunks],
            "pre_bwd_ms": [timed(bwd, c) for c in chunks]}


def measure_general_n(N: int, stream, torch) -> dict:
    """One mHC step (pre fwd, post fwd, post bwd, pre bwd with the h_post_bda dX term) at stream counts
    other than 4, on the kernels templated on n: same token count as the headline workload, a width
    that keeps the residual near 0.5 GB, synthetic N(0,1) bf16 inputs, W ~ N(0, 0.02), the same
    per-channel scale as the layer stand-in.  As for the headline: two copies of the residual
    alternate between steps, HIP events bracket every phase, and the mHC time is the sum of the four
    mHC phases (ms_per_step; ms_per_step_incl_layer adds the layer stand-in's two scale kernels).
    Mean of 5 event-timed steps after one warm-up; GB/s on each boundary tensor once per phase,
    (16 n + 10) C bytes per token, over the mHC time."""
    from mhc_hyper_connection_proj_amd import binding as B
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(5)
    res = {}
    for n, C in ((2, 7168), (8, 2048)):
        Xs = [torch.randn(N, n, C, device=dev, generator=gen).to(torch.bfloat16)]
        Xs.append(Xs[0].clone())
        G = torch.randn(N, n, C, device=dev, generator=gen).to(torch.bfloat16)
        W = torch.randn(n * C, n * n + 2 * n, device=dev, generator=gen) * 0.02
        s = torch.rand(C, device=dev, generator=gen).to(torch.bfloat16) + 0.5
        st = {}

        def pre_fwd():
            st["f"] = B.mhc_pre_fwd(st["X"], W)

        def layer():
            st["x"] = st["f"]["agg"] * s

        def post_fwd():
            B.mhc_h_post_bda_fwd(st["X"], st["f"]["H_res"], st["f"]["H_post"], st["x"])

        def post_bwd():
            f = st["f"]
            _, st["dHr"], st["dHp"], st["dx"], _ = B.mhc_h_post_bda_bwd(G, st["X"], f["H_res"], f["H_post"],
                                                                         st["x"], want_dX=False)

        def layer_bwd():
            st["g"] = st["dx"] * s

        def pre_bwd():
            f = st["f"]
            B.mhc_pre_bwd(st["g"], st["dHp"], st["dHr"], st["X"], W, f["saved"], f["H_pre"], f["H_post"],
                          f["H_res_logits"], post_G=G, post_H_res=f["H_res"])

        seq = [("pre_fwd", pre_fwd, True), ("layer", layer, False), ("post_fwd", post_fwd, True),
               ("post_bwd", post_bwd, True), ("layer_bwd", layer_bwd, False), ("pre_bwd", pre_bwd, True)]
        st["X"] = Xs[0]
        for _, fn, _ in seq:
            fn()
        torch.cuda.synchronize()
        steps = 5
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)] for _ in range(steps)]
        for k in range(steps):
            st["X"] = Xs[(k + 1) % 2]
            evs[k][0].record(stream)
            for i, (_, fn, _) in enumerate(seq):
                fn()
                evs[k][i + 1].record(stream)
        torch.cuda.synchronize()
        ph = {name: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
              for i, (name, _, _) in enumerate(seq)}
        ms = sum(ph[name] for name, _, m in seq if m)
        gbs = (16 * n + 10) * C * N / (ms * 1e-3) / 1e9
        res[f"n{n}_C{C}"] = {"ms_per_step": ms, "ms_per_step_incl_layer": sum(ph.values()),
                             "phases_ms": ph, "tokens_per_s": N / (ms * 1e-3), "achieved_gbs": gbs,
                             "frac": gbs / HBM_PEAK_GBS}
        del Xs, G, W, st
    return res


def measure_configs(stream, torch) -> dict:
    """The other stated workloads at their full sizes (seeded synthetic inputs from synth): batched
    Sinkhorn fwd + bwd (1,048,576 4x4 matrices), the pre forward (32768 tokens, C = 4096) and the
    h_post_bda forward + backward with bias (32768 tokens, C = 4096).  Mean of 5 event-timed calls
    after one warm-up; algorithmic bytes: Sinkhorn 128 + 192 bytes per matrix, pre forward
    10C + 260 per token (X read; agg, H, logits, saved written), h_post_bda 18C + 80 (fwd) and
    28C + 160 (bwd with dX, dx, dH and dbias) per token, bias and dbias once.  The h_post_bda leg's
    H_res is the library's 20-iteration Sinkhorn of N(0,1) logits and its H_post 2 sigmoid(N(0,1)),
    as the workload states."""
    from mhc_hyper_connection_proj_amd import binding as B, synth
    dev = torch.device("cuda", 0)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))

    res = {}
    w = synth.WORKLOADS["sinkhorn_batched"]
    L, dH = to_dev(synth.tensor(w, "L")), to_dev(synth.tensor(w, "dH"))
    ms_f = timed(lambda: B.mhc_sinkhorn_fwd(L, w.iters, w.eps))
    ms_b = timed(lambda: B.mhc_sinkhorn_bwd(dH, L, w.iters, w.eps))
    M = w.tokens
    res["sinkhorn_batched"] = {"matrices": M, "fwd_ms": ms_f, "bwd_ms": ms_b,
                               "matrices_per_s": M / ((ms_f + ms_b) * 1e-3),
                               "achieved_gbs": 320 * M / ((ms_f + ms_b) * 1e-3) / 1e9,
                               "frac": 320 * M / ((ms_f + ms_b) * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del L, dH
    w = synth.WORKLOADS["pre_fwd"]
    N, C = w.tokens, w.C
    X, W = to_dev(synth.tensor(w, "X")), to_dev(synth.tensor(w, "W"))
    ms = timed(lambda: B.mhc_pre_fwd(X, W, None, None, w.rms_eps, w.iters, w.eps))
    byt = (10 * C + 260) * N
    res["pre_fwd"] = {"tokens": N, "C": C, "ms": ms, "tokens_per_s": N / (ms * 1e-3),
                      "achieved_gbs": byt / (ms * 1e-3) / 1e9, "frac": byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del X, W
    w = synth.WORKLOADS["post_bda"]
    N, C = w.tokens, w.C
    X, G, x, b = (to_dev(synth.tensor(w, t)) for t in ("X", "G", "x", "bias"))
    # as stated: H_res doubly stochastic by 20 Sinkhorn iterations on N(0,1) logits (the library's
    # Sinkhorn), H_post = 2 sigmoid(N(0,1))
    Hr = B.mhc_sinkhorn_fwd(to_dev(synth.tensor(w, "L")), w.iters, w.eps)
    Hp = 2.0 * torch.sigmoid(to_dev(synth.tensor(w, "Hpost_logits")))
    ms_f = timed(lambda: B.mhc_h_post_bda_fwd(X, Hr, Hp, x, b))
    ms_b = timed(lambda: B.mhc_h_post_bda_bwd(G, X, Hr, Hp, x, b))
    byt = ((18 * C + 80) + (28 * C + 160)) * N + 4 * C
    res["post_bda_fwd_bwd"] = {"tokens": N, "C": C, "fwd_ms": ms_f, "bwd_ms": ms_b,
                               "tokens_per_s": N / ((ms_f + ms_b) * 1e-3),
                               "achieved_gbs": byt / ((ms_f + ms_b) * 1e-3) / 1e9,
                               "frac": byt / ((ms_f + ms_b) * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return res


def measure_ceilings(lib, L, sp, stream, torch, nbytes: int) -> dict:
    """Practical memory rates of this GPU at the workload's shape (mhc_bandwidth_probe over buffers of
    the residual's size, three rotated so that no call finds its input in the 256 MB Infinity Cache):
    read only and copy (read + write bytes), with default and non-temporal loads; and the re-read of
    one 256 MB buffer, which stays in the Infinity Cache.  Median of 8 event-timed calls."""
    dev = torch.device("cuda", 0)
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(3)]
    sink = torch.empty(4096, dtype=torch.uint8, device=dev)

    def med(fn, reps=8):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))

    res = {"bytes": nbytes}
    for name, kind in (("read", L.MHC_PROBE_READ), ("read_nt", L.MHC_PROBE_READ | L.MHC_PROBE_NONTEMPORAL),
                       ("copy", L.MHC_PROBE_COPY), ("copy_nt", L.MHC_PROBE_COPY | L.MHC_PROBE_NONTEMPORAL)):
        k = [0]
        copy = kind & L.MHC_PROBE_COPY

        def fn():
            src, dst = bufs[k[0] % 3], (bufs[(k[0] + 1) % 3] if copy else sink)
            L.check(lib.mhc_bandwidth_probe(sp, kind, src.data_ptr(), dst.data_ptr(), nbytes))
            k[0] += 1
        ms = med(fn)
        gbs = (2 if copy else 1) * nbytes / (ms * 1e-3) / 1e9
        res[name + "_gbs"] = gbs
        res[name + "_frac"] = gbs / HBM_PEAK_GBS
    small = 256 << 20
    ms = med(lambda: L.check(lib.mhc_bandwidth_probe(sp, L.MHC_PROBE_READ | L.MHC_PROBE_NONTEMPORAL,
                                                     bufs[0].data_ptr(), sink.data_ptr(), small)))
    res["reread_256MiB_nt_gbs"] = small / (ms * 1e-3) / 1e9
    del bufs
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, X, W, s, G, budget_s: float) -> dict:
    """Time the fp64 oracle, as written, on the workload's tokens: the whole mHC fwd + bwd chain (with
    the layer's scale) on chunks of 16 tokens, first on one thread, then on a pool of threads (the
    oracle is C behind ctypes, which releases the GIL) sized to this process's CPU share, at most 16.
    Each leg runs for about budget_s / 2 seconds on its own tokens."""
    import oracle as O
    from concurrent.futures import ThreadPoolExecutor

    O._lib()
    C = w.C
    Wd = W.astype(np.float64)
    sd = O.bf16_bits_to_f64(s)

    def chain(t0, n):
        sl = slice(t0, t0 + n)
        Xc = O.bf16_bits_to_f64(X[sl]); Gc = O.bf16_bits_to_f64(G[sl])
        f = O.pre_fwd(Xc, Wd, eps_rms=w.rms_eps, iters=w.iters, eps=w.eps)
        x = O.round_f64_to_bf16(O.round_f64_to_bf16(f["agg"]) * sd)
        O.h_post_bda_fwd(Xc, f["H_res"], f["H_post"], x, None)
        dX, dHr, dHp, dx, _ = O.h_post_bda_bwd(Gc, Xc, f["H_res"], f["H_post"], x, None)
        g = O.round_f64_to_bf16(O.round_f64_to_bf16(dx) * sd)
        O.pre_bwd(g, dHp, dHr, Xc, Wd, eps_rms=w.rms_eps, iters=w.iters, eps=w.eps)
        return n

    chunk, leg = 16, budget_s / 2
    n1, t_used = 0, 0.0
    while t_used < leg and n1 + chunk <= X.shape[0]:
        t0 = time.perf_counter()
        chain(n1, chunk)
        t_used += time.perf_counter() - t0
        n1 += chunk
    single = n1 / t_used
    try:
        share = len(os.sched_getaffinity(0))
    except AttributeError:
        share = os.cpu_count() or 1
    threads = max(1, min(16, share))
    nchunks = X.shape[0] // chunk
    nt, t0 = 0, time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while time.perf_counter() - t0 < leg:  # the pool walks the workload's chunks, wrapping around
            base = n1 // chunk + nt // chunk
            nt += sum(ex.map(lambda i: chain(((base + i) % nchunks) * chunk, chunk), range(threads)))
    t_pool = time.perf_counter() - t0
    return {"value": nt / t_pool, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{nt} tokens of the workload (C={C}) from token {n1} on, wrapping, full mHC fwd+bwd chain "
                      f"incl. layer scale, fp64, {t_pool:.1f} s on {threads} threads",
            "cpu_model": cpu_model(), "cpu_share": share,
            "single_thread": {"value": single, "unit": "tokens/s", "cores": 1,
                              "sample": f"first {n1} tokens, {t_used:.1f} s on one thread"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=None, help="override token count (testing only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a 1 GiB device copy (for HBM counter calibration under rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over tokens with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    from mhc_hyper_connection_proj_amd import _lib, synth
    from mhc_hyper_connection_proj_amd._lib import MHC_BF16

    lib = _lib.lib()
    w = synth.WORKLOADS["full_layer"]
    N = args.tokens or w.tokens
    C, n, K = w.C, w.n, 4 * w.C
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    X = synth.tensor(w, "X", tokens=N)
    W = synth.tensor(w, "W")
    s = synth.tensor(w, "scale")
    G = synth.tensor(w, "G", tokens=N)
    Xd, Wd, sd, Gd = to_dev(X), to_dev(W), to_dev(s), to_dev(G)
    # Consecutive steps use two copies of the residual (same values, other
    # addresses): a step then cannot find the previous step's X in the 256 MB
    # Infinity Cache, as in a model where every layer has its own residual.
    Xcopies = [Xd, Xd.clone()]
    cur = {"X": Xd}

    f32 = torch.float32
    e = lambda *shape, dt=f32: torch.empty(*shape, dtype=dt, device=dev)
    bf = torch.bfloat16
    H_pre, H_post, H_res, L, saved = e(N, 4), e(N, 4), e(N, 4, 4), e(N, 4, 4), e(N, 32)
    agg, x, out, dx, g = e(N, C, dt=bf), e(N, C, dt=bf), e(N, 4, C, dt=bf), e(N, C, dt=bf), e(N, C, dt=bf)
    dX, dHr, dHp = e(N, 4, C, dt=bf), e(N, 4, 4), e(N, 4)
    dW, da, db = e(K, 24), e(3), e(24)
    ws_f = lib.mhc_pre_fwd_workspace_size(N, n, C, MHC_BF16)
    ws_b = lib.mhc_pre_bwd_workspace_size(N, n, C, MHC_BF16)
    ws_p = lib.mhc_h_post_bda_bwd_workspace_size(N, n, C, MHC_BF16, 0)
    wsf, wsb = e(max(ws_f, 16), dt=torch.uint8), e(max(ws_b, 16), dt=torch.uint8)
    wsp = e(max(ws_p, 16), dt=torch.uint8)
    P = lambda t: t.data_ptr()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def pre_fwd():
        _lib.check(lib.mhc_pre_fwd(sp, N, n, C, MHC_BF16, P(cur["X"]), P(Wd), None, None, w.rms_eps, w.iters, w.eps,
                                   P(H_pre), P(H_post), P(H_res), P(L), P(saved), P(agg), P(wsf), ws_f))

    def post_fwd():
        _lib.check(lib.mhc_h_post_bda_fwd(sp, N, n, C, MHC_BF16, P(cur["X"]), P(H_res), P(H_post), P(x), None, P(out)))

    def post_bwd():
        _lib.check(lib.mhc_h_post_bda_bwd(sp, N, n, C, MHC_BF16, P(Gd), P(cur["X"]), P(H_res), P(H_post), P(x), None,
                                          None, P(dHr), P(dHp), P(dx), None, P(wsp), ws_p))

    def pre_bwd():
        _lib.check(lib.mhc_pre_bwd(sp, N, n, C, MHC_BF16, P(g), P(dHp), P(dHr), P(cur["X"]), P(Wd), None, P(saved),
                                   P(H_pre), P(H_post), P(L), w.iters, w.eps, P(Gd), P(H_res), P(dX), 0, P(dW),
                                   P(da), P(db), None, None, P(wsb), ws_b))

    def layer_fwd():
        torch.mul(agg, sd, out=x)

    def layer_bwd():
        torch.mul(dx, sd, out=g)

    seq = [("pre_fwd", pre_fwd, True), ("layer_fwd", layer_fwd, False), ("post_fwd", post_fwd, True),
           ("post_bwd", post_bwd, True), ("layer_bwd", layer_bwd, False), ("pre_bwd", pre_bwd, True)]

    if args.copy_calib:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for it in range(args.warmup):
        cur["X"] = Xcopies[it % 2]
        for _, fn, _ in seq:
            fn()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)] for _ in range(args.steps)]
    # the dX / dW kernel inside mhc_pre_bwd is timed by events that the
    # library records around its launch (mhc_set_kernel_events); torch creates
    # an event's handle at its first record, so each is recorded once here
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for pair in kev:
        for ev in pair:
            ev.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.steps):
        cur["X"] = Xcopies[(args.warmup + st) % 2]
        evs[st][0].record(stream)
        for i, (name, fn, _) in enumerate(seq):
            if name == "pre_bwd":
                _lib.check(lib.mhc_set_kernel_events(_lib.MHC_KERNEL_PROJ_BWD_DXDW, kev[st][0]._as_parameter_,
                                                     kev[st][1]._as_parameter_))
            fn()
            if name == "pre_bwd":
                _lib.check(lib.mhc_set_kernel_events(0, None, None))
            evs[st][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    phase_ms = {name: [] for name, _, _ in seq}
    for st in range(args.steps):
        for i, (name, _, _) in enumerate(seq):
            phase_ms[name].append(evs[st][i].elapsed_time(evs[st][i + 1]))
    mean = {k: float(np.mean(v)) for k, v in phase_ms.items()}
    mhc_ms = sum(mean[k] for k, _, m in seq if m)
    step_ms = sum(mean.values())

    ceilings = measure_ceilings(lib, _lib, sp, stream, torch, N * n * C * 2)
    projection_choice = measure_projection_choice(lib, _lib, sp, stream, torch, cur["X"], Wd, N, n, C)
    norm_bwd_fusion = measure_norm_bwd_fusion(lib, _lib, sp, stream, torch, N, n, C, cur["X"], Wd, Gd, H_res, agg, g,
                                              saved, H_pre, H_post, L, dHp, dHr)
    variants = measure_variants(lib, _lib, sp, N, n, C, cur["X"], Gd, H_res, H_post, x, g, out, dX, dHr, dHp, dx,
                                stream, torch)
    reread = measure_reread_chunks(lib, _lib, sp, stream, torch, Xcopies, Wd, Gd,
                                   {"H_pre": H_pre, "H_post": H_post, "H_res": H_res, "L": L, "saved": saved,
                                    "agg": agg, "g": g, "dHp": dHp, "dHr": dHr, "dX": dX, "dW": dW, "da": da,
                                    "db": db}, N, n, C, w.rms_eps, w.iters, w.eps)
    general_n = measure_general_n(N, stream, torch)
    configs = measure_configs(stream, torch)

    led = ledger_bytes_per_token(C, N)
    tot_bytes = led["total"] * N
    gbs = tot_bytes / (mhc_ms * 1e-3) / 1e9

    # dominant kernel: the dX / dW kernel of the pre backward, timed alone
    kname = "proj_bwd_mfma16_kernel"
    k_ms = float(np.mean([kev[st][0].elapsed_time(kev[st][1]) for st in range(args.steps)]))
    k_bytes = led["dxdw_kernel"] * N
    k_gbs = k_bytes / (k_ms * 1e-3) / 1e9
    traffic = pmc_traffic("proj_bwd_dxdw_full_layer_pmc.txt", ["mhc_hyper_connection_proj_amd/csrc/proj.hip",
                                                               "mhc_hyper_connection_proj_amd/csrc/device.h",
                                                               "mhc_hyper_connection_proj_amd/csrc/ring.h"])
    # the h_post_bda backward (one kernel, the whole post_bwd phase), for context
    p_bytes = led["post_bwd"] * N
    p_gbs = p_bytes / (mean["post_bwd"] * 1e-3) / 1e9
    p_traffic = pmc_traffic("h_post_bda_bwd_full_layer_pmc.txt", ["mhc_hyper_connection_proj_amd/csrc/streams.hip",
                                                                  "mhc_hyper_connection_proj_amd/csrc/device.h"])

    res = {
        "metric": METRIC,
        "value": N / (mhc_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": mhc_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "full_layer: B=4 T=4096 n=4 C=7168 bf16 residual, fp32 W [28672,24], "
                               "Sinkhorn 20 iters eps=1e-6, layer = per-channel bf16 scale, no bias",
                   "tokens": N, "n": n, "C": C, "parallelism": "single GPU"},
        "achieved_gbs": gbs,
        "hbm_frac": gbs / HBM_PEAK_GBS,
        "ledger_bytes_per_token": led["total"],
        "ledger": "74C+1336 bytes per token: every boundary tensor once per phase, the h_post_bda residual "
                  "gradient formed inside the pre backward from G (so dX is written once), W and dW amortised",
        "hbm_frac_82C_ledger": (82 * C + 1232) * N / (mhc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "ceilings": ceilings,
        "projection_mfma_vs_fma": projection_choice,
        "pre_rmsnorm_bwd": norm_bwd_fusion,
        "phases_ms": mean,
        "ms_per_step_incl_layer": step_ms,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": k_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": k_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": k_bytes, "avg_launch_ms": k_ms},
        "roofline_h_post_bda_bwd": {"bound": "hbm", "kernel": "h_post_bda_bwd_kernel", "achieved": p_gbs,
                                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": p_gbs / HBM_PEAK_GBS,
                                    "traffic": p_traffic, "algorithmic_bytes_per_launch": p_bytes,
                                    "avg_launch_ms": mean["post_bwd"]},
        "variants": variants,
        "reread_chunks": reread,
        "general_n": general_n,
        "configs": configs,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, X, W, s, G, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
