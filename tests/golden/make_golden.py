"""Write the oracle regression fixtures in this folder (run from the repository root:
``python tests/golden/make_golden.py``).

The pages print no worked numeric example for this path, so no fixture here
holds a value taken from them.  Each fixture is a tiny seeded case evaluated
by the fp64 oracle (this script calls nothing but ``oracle``); the test that
reads them re-evaluates the oracle and flags any change of its arithmetic.
The oracle's correctness is established separately, by the pins in
``tests/test_oracle_pins.py``.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402


def cases():
    rng = np.random.default_rng(20261202)
    N, n, C = 3, 4, 8
    X = rng.standard_normal((N, n, C))
    W = rng.standard_normal((n * C, n * n + 2 * n)) * 0.2
    G = rng.standard_normal((N, n, C))
    x = rng.standard_normal((N, C))
    bias = rng.standard_normal(C) * 0.1
    gamma = rng.uniform(0.5, 1.5, C)
    dy = rng.standard_normal((N, C))
    L = rng.standard_normal((N, n, n)) * 1.5
    dH = rng.standard_normal((N, n, n))
    yield "proj_rms_h", "Megatron Core fused_mhc_kernels, _torch_proj_rms_compute_h", dict(X=X, W=W), \
        lambda: (lambda p: dict(H_pre=p.H_pre, H_post=p.H_post, L=p.L, r=p.r))(O.proj_rms_h(X, W))
    yield "sinkhorn", "rwkv-ops mhu_ffi.cu, Sinkhorn Knopp FFI (20 iterations, eps 1e-6)", dict(L=L, dH=dH), \
        lambda: dict(H=O.sinkhorn_fwd(L, 20, 1e-6), dL=O.sinkhorn_bwd(dH, L, 20, 1e-6))
    H_res = O.sinkhorn_fwd(L, 20, 1e-6)
    H_post = 2 / (1 + np.exp(-rng.standard_normal((N, n))))
    yield "h_post_bda", "Megatron Core fused_mhc_kernels, h_post_bda and _torch_h_post_bda_bwd", \
        dict(X=X, H_res=H_res, H_post=H_post, x=x, bias=bias, G=G), \
        lambda: (lambda f, b: dict(out=f, dX=b[0], dH_res=b[1], dH_post=b[2], dx=b[3], dbias=b[4]))(
            O.h_post_bda_fwd(X, H_res, H_post, x, bias), O.h_post_bda_bwd(G, X, H_res, H_post, x, bias))
    H_pre = 1 / (1 + np.exp(-rng.standard_normal((N, n))))
    yield "h_aggregate", "Megatron Core fused_mhc_kernels, h_aggregate and _torch_h_aggregate_bwd", \
        dict(X=X, H_pre=H_pre, g=x), \
        lambda: (lambda f, b: dict(agg=f, dX=b[0], dH_pre=b[1]))(O.h_aggregate_fwd(X, H_pre),
                                                                 O.h_aggregate_bwd(x, X, H_pre))
    yield "rmsnorm", "rwkv-ops mhu_ffi.cu, RMSNorm FFI; RL-Kernel PR #383 rmsnorm_residual gain", \
        dict(x=x, gamma=gamma, dy=dy), \
        lambda: (lambda f, b: dict(y=f[0], dx=b[0], dgamma=b[1]))(O.rmsnorm_fwd(x, gamma, 1e-6),
                                                                  O.rmsnorm_bwd(dy, x, gamma, 1e-6))
    yield "pre_bwd", "composition: h_aggregate bwd + Sinkhorn bwd + projection bwd (Megatron fused_add_3)", \
        dict(g=x, dH_post=H_post, dH_res=dH, X=X, W=W), \
        lambda: (lambda r: dict(dX=r["dX"], dW=r["dW"], dalpha=r["dalpha"], dhbias=r["dhbias"]))(
            O.pre_bwd(x, H_post, dH, X, W))


def main():
    for name, cite, inputs, fn in cases():
        out = fn()
        rec = {"source": cite, "producer": "tests/golden/make_golden.py (fp64 oracle)",
               "inputs": {k: np.asarray(v).tolist() for k, v in inputs.items()},
               "outputs": {k: np.asarray(v).tolist() for k, v in out.items()}}
        with open(os.path.join(HERE, f"{name}.json"), "w") as f:
            json.dump(rec, f, indent=0)
        print("wrote", name)


if __name__ == "__main__":
    main()
