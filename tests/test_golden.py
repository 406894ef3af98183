"""Checks against the numbers the pages print (tests/golden/pages_values.json)
and a regression guard on the oracle's own outputs (tests/golden/oracle_tiny.json)."""
import json
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_fp16_score_matrix_size_matches_page():
    """FA page section 3: an fp16 S for B=1, H=32, N=8192 takes 4096 MiB (2BHN^2 bytes)."""
    g = _load("pages_values.json")["score_matrix_mib_fp16"]["value"]
    w = workloads.ATTN["C4"]
    assert (w.B, w.H, w.N) == (g["B"], g["H"], g["N"])
    assert 2 * w.B * w.H * w.N * w.N / 2 ** 20 == g["MiB"]


def test_flop_model_matches_page():
    """FA page section 1: non-causal 4BHN^2D, causal about 2BHN^2D."""
    g = _load("pages_values.json")["flop_model"]["value"]
    assert workloads.attn_flops(1, 32, 8192, 128, True) == g["causal_factor"] * 32 * 8192 ** 2 * 128
    assert workloads.attn_flops(4, 32, 4095, 64, False) == g["noncausal_factor"] * 4 * 32 * 4095 ** 2 * 64


def test_workload_geometry_matches_page():
    g = _load("pages_values.json")["fa_geometry"]["value"]
    for name in ("C2", "C3", "C4"):
        w = workloads.ATTN[name]
        assert (w.B, w.H, w.D, w.causal) == (g["B"], g["H"], g["D"], g["causal"])
        assert w.N in g["N"]
    s = _load("pages_values.json")["softmax_boundary_shape"]["value"]
    assert (workloads.SOFTMAX["R1"].M, workloads.SOFTMAX["R1"].N) == (s["M"], s["N"])


def test_tolerances_cover_the_pages_observed_errors():
    """The fp16 output tolerance (4e-3) sits above the page's observed fp16 FA-vs-math max-abs
    error, and the row-softmax tolerance equals the study's pass threshold."""
    from tests import tolerances
    g = _load("pages_values.json")
    assert tolerances.ATTN_O["f16"] > g["fp16_fa_vs_math_max_abs"]["value"]
    assert tolerances.SOFTMAX_Y == g["softmax_pass_threshold"]["value"]
    assert max(g["softmax_fp32_error_magnitude"]["value"]) < tolerances.SOFTMAX_Y


def test_oracle_regression_fixture():
    """Oracle + input recipe reproduce the stored values bit for bit."""
    fx = _load("oracle_tiny.json")
    for c in fx["attn"]:
        q, k, v = workloads.attn_inputs(c["B"], c["H"], c["N"], c["D"], c["dtype"], c["seed"])
        o, lse = oracle.attn_fwd(q, k, v, c["causal"], nthreads=2)
        assert o.reshape(-1).tolist() == c["o"]
        assert lse.reshape(-1).tolist() == c["lse"]
    s = fx["softmax"][0]
    x = workloads.softmax_inputs(s["M"], s["N"], seed=s["seed"], last=s["last"])
    assert oracle.row_softmax(x).reshape(-1).tolist() == s["y"]
    assert np.isfinite(np.array(s["y"])).all()
