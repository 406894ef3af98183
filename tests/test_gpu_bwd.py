"""GPU parity of attn_bwd (through the C ABI) against the FP64 backward oracle.

The GPU backward runs on the GPU forward's O and LSE (the product path: forward
then backward); the oracle recomputes everything from Q, K, V and dO.  dQ, dK,
dV and the workspace are NaN-prefilled.  Tolerance (tests/tolerances.py):
max |G - G_ref| <= 4u * max(1, max |G_ref|), u the dtype's unit roundoff.
"""
import numpy as np
import pytest
import torch

import oracle
import online_softmax_causal_amd as osc
import workloads
from tests import tolerances
from tests.test_gpu_attn import dev

pytestmark = pytest.mark.gpu


def run_bwd(q, k, v, do, causal, dtype):
    d = dev()
    B, H, N, D = q.shape
    qd, kd, vd, dod = (t.to(d) for t in (q, k, v, do))
    o = torch.empty((B, H, N, D), dtype=torch.float32, device=d)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=d)
    osc.attn_fwd(qd, kd, vd, o, lse, B, H, N, D, causal, dtype)
    grads = [torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device=d) for _ in range(3)]
    need = osc.attn_bwd_workspace(B, H, N)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=d)
    osc.attn_bwd(qd, kd, vd, o, lse, dod, *grads, B, H, N, D, causal, dtype, ws, need)
    torch.cuda.synchronize()
    return [g.cpu().double().numpy() for g in grads]


def check(name, got, ref, dtype):
    for label, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.isfinite(g).all(), "%s: non-finite %s" % (name, label)
        err = np.abs(g - r).max()
        tol = tolerances.BWD_REL[dtype] * max(1.0, np.abs(r).max())
        print("%s %s: max err %.3e  tol %.3e" % (name, label, err, tol), flush=True)
        assert err <= tol, "%s: %s error %.3e > %.3e" % (name, label, err, tol)


SMALL = [
    # (B, H, N, D): single row, tile edges (32, 64, 128), ragged lengths
    (1, 1, 1, 128), (1, 2, 31, 64), (1, 1, 64, 128), (2, 1, 65, 64), (1, 2, 127, 128),
    (1, 1, 129, 64), (1, 2, 200, 128), (2, 1, 333, 64), (1, 1, 513, 128),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dN%dD%d" % s)
def test_small_shapes_match_oracle(shape, causal, dtype):
    B, H, N, D = shape
    seed = 9000 + 3 * N + D + (1 if causal else 0)
    q, k, v, do = workloads.bwd_inputs(B, H, N, D, dtype, seed, sigma_qk=1.5)
    name = "bwd %s %s B%d H%d N%d D%d seed %d" % ("causal" if causal else "full", dtype, B, H, N, D, seed)
    print("running", name, flush=True)
    got = run_bwd(q, k, v, do, causal, dtype)
    check(name, got, oracle.attn_bwd(q, k, v, do, causal), dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_large_logits(dtype):
    """Q, K ~ N(0, 3^2) (the C3 recipe): peaked rows, |s| up to ~30."""
    q, k, v, do = workloads.bwd_inputs(1, 2, 700, 128, dtype, 9101, sigma_qk=3.0)
    print("running bwd large logits", dtype, flush=True)
    got = run_bwd(q, k, v, do, True, dtype)
    check("bwd large logits %s" % dtype, got, oracle.attn_bwd(q, k, v, do, True), dtype)


def test_deterministic():
    q, k, v, do = workloads.bwd_inputs(1, 3, 777, 128, "f16", 9102)
    print("running bwd determinism", flush=True)
    a = run_bwd(q, k, v, do, True, "f16")
    b = run_bwd(q, k, v, do, True, "f16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_headline_shape_sampled_heads():
    """Causal fp16 B1 H32 N8192 D128 (the benchmark's backward workload):
    every element of two heads against the oracle, finiteness everywhere."""
    w = workloads.ATTN["C4"]
    q, k, v, do = workloads.bwd_inputs(w.B, w.H, w.N, w.D, w.dtype, w.seed)
    print("running bwd", w.describe(), flush=True)
    got = run_bwd(q, k, v, do, w.causal, w.dtype)
    heads = [0, w.H - 1]
    ref = oracle.attn_bwd(q, k, v, do, w.causal, heads=heads)
    check("bwd C4 heads %s" % heads, [g.reshape(-1, w.N, w.D)[heads] for g in got], ref, w.dtype)


# ------------------------------------------------- grouped K/V heads (GQA)

def run_bwd_gqa(q, k, v, do, causal, dtype):
    d = dev()
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    qd, kd, vd, dod = (t.to(d) for t in (q, k, v, do))
    o = torch.empty((B, H, N, D), dtype=torch.float32, device=d)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=d)
    osc.attn_fwd_gqa(qd, kd, vd, o, lse, B, H, Hkv, N, D, causal, dtype)
    dq = torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device=d)
    dk = torch.full((B, Hkv, N, D), float("nan"), dtype=torch.float32, device=d)
    dv = torch.full((B, Hkv, N, D), float("nan"), dtype=torch.float32, device=d)
    need = osc.attn_bwd_workspace(B, H, N)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=d)
    osc.attn_bwd_gqa(qd, kd, vd, o, lse, dod, dq, dk, dv, B, H, Hkv, N, D, causal, dtype, ws, need)
    torch.cuda.synchronize()
    return [g.cpu().double().numpy() for g in (dq, dk, dv)]


GQA_SMALL = [
    # (B, H, Hkv, N, D): groups of 2, 3, 4 and 8 (MQA), one row, ragged lengths
    (1, 4, 2, 65, 128), (2, 6, 2, 129, 64), (1, 8, 1, 200, 128), (1, 8, 2, 1, 128),
    (2, 4, 1, 333, 64), (1, 6, 3, 97, 128),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", GQA_SMALL, ids=lambda s: "B%dH%dHkv%dN%dD%d" % s)
def test_gqa_small_shapes_match_oracle(shape, causal, dtype):
    B, H, Hkv, N, D = shape
    seed = 9200 + 7 * N + D + Hkv + (1 if causal else 0)
    q, k, v, do = workloads.bwd_gqa_inputs(B, H, Hkv, N, D, dtype, seed, sigma_qk=1.5)
    name = "bwd gqa %s %s B%d H%d Hkv%d N%d D%d seed %d" % (
        "causal" if causal else "full", dtype, B, H, Hkv, N, D, seed)
    print("running", name, flush=True)
    got = run_bwd_gqa(q, k, v, do, causal, dtype)
    check(name, got, oracle.attn_bwd_gqa(q, k, v, do, causal), dtype)


def test_gqa_with_one_head_per_group_equals_attn_bwd():
    q, k, v, do = workloads.bwd_inputs(1, 3, 200, 128, "bf16", 9201)
    print("running bwd gqa Hkv = H", flush=True)
    a = run_bwd_gqa(q, k, v, do, True, "bf16")
    b = run_bwd(q, k, v, do, True, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_gqa_deterministic():
    q, k, v, do = workloads.bwd_gqa_inputs(1, 8, 2, 500, 128, "f16", 9202)
    print("running bwd gqa determinism", flush=True)
    a = run_bwd_gqa(q, k, v, do, True, "f16")
    b = run_bwd_gqa(q, k, v, do, True, "f16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_gqa_benchmark_shape_sampled():
    """Causal fp16 B1 H32 Hkv8 N8192 D128 (the G1 shape): dK, dV of one K/V
    head and dQ of its four query heads against the oracle, finiteness of all."""
    w = workloads.GQA["G1"]
    q, k, v, do = workloads.bwd_gqa_inputs(w.B, w.H, w.Hkv, w.N, w.D, w.dtype, w.seed)
    print("running bwd gqa", w.describe(), flush=True)
    got = run_bwd_gqa(q, k, v, do, w.causal, w.dtype)
    for x in got:
        assert np.isfinite(x).all()
    j = w.Hkv - 1
    g = w.H // w.Hkv
    rq, rk, rv = oracle.attn_bwd_gqa(q, k, v, do, w.causal, kv_heads=[j])
    check("bwd G1 kv head %d" % j,
          [got[0].reshape(-1, w.N, w.D)[j * g:(j + 1) * g], got[1].reshape(-1, w.N, w.D)[[j]],
           got[2].reshape(-1, w.N, w.D)[[j]]], [rq, rk, rv], w.dtype)
