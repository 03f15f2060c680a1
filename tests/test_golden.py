"""Oracle regression fixtures (tests/golden/*.json): the oracle, re-run on each
stored input, must reproduce the stored outputs to rounding.

The fixtures were written by tests/golden/make_golden.py from the oracle itself
(the pages print no worked values for this path), so they guard against
unintended changes of the oracle's arithmetic; its correctness rests on the
pins in test_oracle_pins.py.  A deliberate change of the oracle regenerates
them and names the passage that justifies it.
"""
import glob
import json
import os

import numpy as np
import pytest

import oracle as O

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FILES = sorted(glob.glob(os.path.join(HERE, "*.json")))


def _run(name, a):
    if name == "proj_rms_h":
        p = O.proj_rms_h(a["X"], a["W"])
        return dict(H_pre=p.H_pre, H_post=p.H_post, L=p.L, r=p.r)
    if name == "sinkhorn":
        return dict(H=O.sinkhorn_fwd(a["L"], 20, 1e-6), dL=O.sinkhorn_bwd(a["dH"], a["L"], 20, 1e-6))
    if name == "h_post_bda":
        b = O.h_post_bda_bwd(a["G"], a["X"], a["H_res"], a["H_post"], a["x"], a["bias"])
        return dict(out=O.h_post_bda_fwd(a["X"], a["H_res"], a["H_post"], a["x"], a["bias"]), dX=b[0],
                    dH_res=b[1], dH_post=b[2], dx=b[3], dbias=b[4])
    if name == "h_aggregate":
        b = O.h_aggregate_bwd(a["g"], a["X"], a["H_pre"])
        return dict(agg=O.h_aggregate_fwd(a["X"], a["H_pre"]), dX=b[0], dH_pre=b[1])
    if name == "rmsnorm":
        y, _ = O.rmsnorm_fwd(a["x"], a["gamma"], 1e-6)
        dx, dg = O.rmsnorm_bwd(a["dy"], a["x"], a["gamma"], 1e-6)
        return dict(y=y, dx=dx, dgamma=dg)
    if name == "pre_bwd":
        r = O.pre_bwd(a["g"], a["dH_post"], a["dH_res"], a["X"], a["W"])
        return dict(dX=r["dX"], dW=r["dW"], dalpha=r["dalpha"], dhbias=r["dhbias"])
    raise KeyError(name)


def test_golden_files_present():
    names = {os.path.splitext(os.path.basename(f))[0] for f in FILES}
    assert {"proj_rms_h", "sinkhorn", "h_post_bda", "h_aggregate", "rmsnorm", "pre_bwd"} <= names


@pytest.mark.parametrize("path", FILES, ids=lambda p: os.path.basename(p))
def test_oracle_reproduces_golden(path):
    rec = json.load(open(path))
    assert rec["source"] and rec["producer"].startswith("tests/golden/make_golden.py")
    a = {k: np.asarray(v, dtype=np.float64) for k, v in rec["inputs"].items()}
    got = _run(os.path.splitext(os.path.basename(path))[0], a)
    for k, want in rec["outputs"].items():
        np.testing.assert_allclose(got[k], np.asarray(want), rtol=1e-12, atol=1e-14, err_msg=k)
