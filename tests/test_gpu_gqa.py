"""GPU parity of attn_fwd_gqa (grouped K/V heads, through the C ABI) against the
FP64 oracle, and agreement with attn_fwd on K/V heads expanded per query head.

Query head h reads K/V head h // (H / Hkv) ("CUDA KV Cache: paged storage and
long-context decode", section 3).  Tolerances as for attn_fwd.
"""
import numpy as np
import pytest
import torch

import oracle
import online_softmax_causal_amd as osc
import workloads
from tests import tolerances
from tests.test_gpu_attn import check, dev

pytestmark = pytest.mark.gpu


def run_gqa(q, k, v, causal, dtype):
    d = dev()
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    o = torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device=d)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=d)
    osc.attn_fwd_gqa(qd, kd, vd, o, lse, B, H, Hkv, N, D, causal, dtype)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def run_expanded(q, k, v, causal, dtype):
    """attn_fwd on K/V copied out to one head per query head (test-side expansion)."""
    d = dev()
    B, H, N, D = q.shape
    g = H // k.shape[1]
    ke = k.repeat_interleave(g, dim=1).contiguous()
    ve = v.repeat_interleave(g, dim=1).contiguous()
    o = torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device=d)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=d)
    osc.attn_fwd(q.to(d), ke.to(d), ve.to(d), o, lse, B, H, N, D, causal, dtype)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


SHAPES = [
    # (B, H, Hkv, N, D): MQA, groups of 2..8, Hkv = H, ragged N
    (1, 4, 1, 100, 128), (2, 8, 2, 257, 64), (1, 6, 3, 129, 128), (1, 4, 4, 65, 64),
    (1, 8, 1, 1, 128), (2, 16, 4, 513, 128), (1, 12, 4, 300, 64),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dKV%dN%dD%d" % s)
def test_gqa_small_shapes_match_oracle(shape, causal, dtype):
    B, H, Hkv, N, D = shape
    seed = 3000 + N * 5 + H * 3 + Hkv + (1 if causal else 0)
    q, k, v = workloads.gqa_inputs(B, H, Hkv, N, D, dtype, seed, sigma_qk=1.5)
    name = "gqa %s %s B%d H%d Hkv%d N%d D%d seed %d" % (
        "causal" if causal else "full", dtype, B, H, Hkv, N, D, seed)
    print("running", name, flush=True)
    o, lse = run_gqa(q, k, v, causal, dtype)
    o_ref, lse_ref = oracle.attn_fwd_gqa(q, k, v, causal)
    check(name, o, lse, o_ref, lse_ref, dtype)


@pytest.mark.parametrize("shape", [(1, 8, 2, 333, 128), (2, 6, 1, 200, 64)],
                         ids=lambda s: "B%dH%dKV%dN%dD%d" % s)
def test_gqa_equals_attn_fwd_on_expanded_heads(shape):
    """Reading the shared K/V head in place gives the same bits as a copied-out K/V."""
    B, H, Hkv, N, D = shape
    q, k, v = workloads.gqa_inputs(B, H, Hkv, N, D, "f16", 3100 + N)
    print("running gqa vs expanded B%d H%d Hkv%d N%d D%d" % shape, flush=True)
    o1, l1 = run_gqa(q, k, v, True, "f16")
    o2, l2 = run_expanded(q, k, v, True, "f16")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_gqa_g2_full_compare():
    w = workloads.GQA["G2"]
    print("running G2", w.describe(), flush=True)
    q, k, v = workloads.workload_inputs(w)
    o, lse = run_gqa(q, k, v, w.causal, w.dtype)
    o_ref, lse_ref = oracle.attn_fwd_gqa(q, k, v, w.causal)
    check("G2", o, lse, o_ref, lse_ref, w.dtype)


def test_gqa_g1_sampled_rows():
    """Full-size grouped workload in the launch configuration the benchmark times."""
    w = workloads.GQA["G1"]
    print("running G1", w.describe(), flush=True)
    q, k, v = workloads.workload_inputs(w)
    o, lse = run_gqa(q, k, v, w.causal, w.dtype)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = workloads.sample_rows(w.B, w.H, w.N, 384, seed=w.seed)
    o_ref, lse_ref = oracle.attn_rows_gqa(q, k, v, w.causal, rows)
    check("G1 sampled", o.reshape(-1, w.D)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, w.dtype)


# Grouped heads on the 8-wave workgroups (B*H*ceil(N/256) >= 512): the small
# shapes above all run the 4-wave ring kernel.  Ragged N; every element
# compared.
WIDE_GQA = [
    # (B, H, Hkv, N, D)
    (1, 256, 32, 500, 128),   # groups of 8, ragged second query tile
    (2, 128, 16, 300, 64),    # groups of 8 at D = 64
    (1, 512, 128, 200, 128),  # groups of 4, one partial query tile
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", WIDE_GQA, ids=lambda s: "B%dH%dKV%dN%dD%d" % s)
def test_gqa_wide_shapes_match_oracle(shape, causal, dtype):
    B, H, Hkv, N, D = shape
    assert B * H * ((N + 255) // 256) >= 512 and Hkv < H
    seed = 3200 + N * 5 + H * 3 + Hkv + (1 if causal else 0)
    q, k, v = workloads.gqa_inputs(B, H, Hkv, N, D, dtype, seed, sigma_qk=1.5)
    name = "wide gqa %s %s B%d H%d Hkv%d N%d D%d seed %d" % (
        "causal" if causal else "full", dtype, B, H, Hkv, N, D, seed)
    print("running", name, flush=True)
    o, lse = run_gqa(q, k, v, causal, dtype)
    o_ref, lse_ref = oracle.attn_fwd_gqa(q, k, v, causal)
    check(name, o, lse, o_ref, lse_ref, dtype)
