"""GPU parity of attn_fwd_splitkv (keys split into segments, partial states in
a caller workspace, then a merge kernel; through the C ABI) against the FP64
oracle.  The merged result is plain attention, so the oracle is attn_fwd_gqa.

The workspace is prefilled with NaN: the merge must read only states the
first kernel wrote.  Tolerances as for attn_fwd.
"""
import numpy as np
import pytest
import torch

import oracle
import online_softmax_causal_amd as osc
import workloads
from tests.test_gpu_attn import check, dev

pytestmark = pytest.mark.gpu


def run_split(q, k, v, causal, dtype, splits, ws=None):
    d = dev()
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    need = osc.attn_fwd_splitkv_workspace(B, H, N, D, causal, splits)
    assert need >= 0
    if ws is None:
        ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device=d)
    else:
        ws.fill_(float("nan"))
    assert ws.numel() * 4 >= need
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    o = torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device=d)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=d)
    osc.attn_fwd_splitkv(qd, kd, vd, o, lse, B, H, Hkv, N, D, causal, dtype, splits, ws,
                         ws.numel() * 4)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy(), need


SHAPES = [
    # (B, H, Hkv, N, D, splits): ragged N, a last segment of a single key,
    # more requested splits than 256-key units, GQA with a split
    (1, 2, 2, 1000, 128, 3), (1, 1, 1, 3000, 64, 4), (2, 3, 3, 777, 128, 16),
    (1, 1, 1, 257, 128, 2), (1, 4, 2, 2048, 64, 8), (1, 2, 1, 1537, 128, 5),
    (1, 1, 1, 64, 128, 4),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dKV%dN%dD%dS%d" % s)
def test_splitkv_small_shapes_match_oracle(shape, causal, dtype):
    B, H, Hkv, N, D, splits = shape
    seed = 5000 + N + 11 * splits + (1 if causal else 0)
    q, k, v = workloads.gqa_inputs(B, H, Hkv, N, D, dtype, seed, sigma_qk=1.5)
    name = "splitkv %s %s B%d H%d Hkv%d N%d D%d splits %d seed %d" % (
        "causal" if causal else "full", dtype, B, H, Hkv, N, D, splits, seed)
    print("running", name, flush=True)
    o, lse, need = run_split(q, k, v, causal, dtype, splits)
    if N > 256:
        assert need > 0, "expected a split for %s" % name
    o_ref, lse_ref = oracle.attn_fwd_gqa(q, k, v, causal)
    check(name, o, lse, o_ref, lse_ref, dtype)


def test_splitkv_reused_workspace_smaller_second_call():
    """One workspace serves two calls in a row, the second smaller."""
    d = dev()
    need = osc.attn_fwd_splitkv_workspace(1, 2, 3000, 128, 1, 6)
    ws = torch.empty((need // 4,), dtype=torch.float32, device=d)
    for (N, splits, seed) in [(3000, 6, 5101), (900, 3, 5102)]:
        q, k, v = workloads.attn_inputs(1, 2, N, 128, "f16", seed)
        print("running splitkv reuse N%d splits %d" % (N, splits), flush=True)
        o, lse, _ = run_split(q, k, v, True, "f16", splits, ws=ws)
        o_ref, lse_ref = oracle.attn_fwd(q, k, v, True)
        check("reuse N%d" % N, o, lse, o_ref, lse_ref, "f16")


def test_splitkv_c2_split_full_compare():
    """C2 (causal fp16 B1 H32 N512 D128) with two segments; every element."""
    w = workloads.ATTN["C2"]
    print("running splitkv 2 segments", w.describe(), flush=True)
    q, k, v = workloads.workload_inputs(w)
    o, lse, need = run_split(q, k, v, w.causal, w.dtype, 2)
    assert need > 0
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.causal)
    check("C2 splitkv", o, lse, o_ref, lse_ref, w.dtype)


def test_splitkv_s1_auto_sampled_rows():
    """S1 (causal fp16 B1 H2 N16384 D128), automatic plan as the benchmark runs it."""
    w = workloads.SPLITKV["S1"]
    print("running splitkv auto", w.describe(), flush=True)
    q, k, v = workloads.workload_inputs(w)
    o, lse, need = run_split(q, k, v, w.causal, w.dtype, 0)
    assert need > 0
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = workloads.sample_rows(w.B, w.H, w.N, 384, seed=w.seed)
    o_ref, lse_ref = oracle.attn_rows(q, k, v, w.causal, rows)
    check("S1 sampled", o.reshape(-1, w.D)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, w.dtype)


def test_splitkv_without_split_equals_attn_fwd():
    """When the plan keeps one segment the call is attn_fwd, bit for bit (no workspace)."""
    w = workloads.ATTN["C3"]
    assert osc.attn_fwd_splitkv_workspace(w.B, w.H, w.N, w.D, w.causal, 1) == 0
    q, k, v = workloads.workload_inputs(w)
    print("running splitkv 1 segment", w.describe(), flush=True)
    d = dev()
    o1, l1, _ = run_split(q, k, v, w.causal, w.dtype, 1)
    o = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=d)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=d)
    osc.attn_fwd(q.to(d), k.to(d), v.to(d), o, lse, w.B, w.H, w.N, w.D, w.causal, w.dtype)
    torch.cuda.synchronize()
    assert np.array_equal(o1, o.cpu().double().numpy())
    assert np.array_equal(l1, lse.cpu().double().numpy())
