"""GPU parity of attn_fwd (HIP, through the C ABI) against the FP64 oracle.

Every case prints what it runs before the GPU call.  Outputs are prefilled
with NaN so an element the kernel fails to write shows up as non-finite.
Tolerances (max-abs): O 4e-3 for fp16 inputs, 1.6e-2 for bf16; LSE 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import online_softmax_causal_amd as osc
import workloads
from tests import tolerances

pytestmark = pytest.mark.gpu


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_gpu(q, k, v, causal, dtype):
    d = dev()
    B, H, N, D = q.shape
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    o = torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device=d)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=d)
    osc.attn_fwd(qd, kd, vd, o, lse, B, H, N, D, causal, dtype)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def check(name, o, lse, o_ref, lse_ref, dtype):
    assert np.isfinite(o).all(), "%s: non-finite O (unwritten or NaN)" % name
    assert np.isfinite(lse).all(), "%s: non-finite LSE" % name
    eo = np.abs(o - o_ref).max()
    el = np.abs(lse - lse_ref).max()
    print("%s: max|dO| %.3e  max|dLSE| %.3e" % (name, eo, el), flush=True)
    assert eo <= tolerances.ATTN_O[dtype], "%s: O error %.3e" % (name, eo)
    assert el <= tolerances.ATTN_LSE, "%s: LSE error %.3e" % (name, el)


SMALL = [
    # (B, H, N, D) -- N spans single rows, tile edges (32, 64, 128, 256) and ragged tails
    (1, 1, 1, 128), (1, 2, 2, 64), (1, 1, 3, 128), (2, 1, 17, 64), (1, 2, 63, 128),
    (1, 1, 64, 64), (1, 3, 65, 128), (1, 1, 127, 64), (1, 1, 129, 128), (1, 2, 255, 64),
    (2, 1, 257, 128), (1, 1, 300, 64), (1, 1, 511, 128), (1, 2, 513, 64), (1, 1, 1000, 128),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dN%dD%d" % s)
def test_small_shapes_match_oracle(shape, causal, dtype):
    B, H, N, D = shape
    seed = 1000 + N * 7 + D + (1 if causal else 0)
    q, k, v = workloads.attn_inputs(B, H, N, D, dtype, seed, sigma_qk=1.5)
    name = "attn %s %s B%d H%d N%d D%d seed %d" % ("causal" if causal else "full", dtype, B, H, N, D, seed)
    print("running", name, flush=True)
    o, lse = run_gpu(q, k, v, causal, dtype)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal)
    check(name, o, lse, o_ref, lse_ref, dtype)


@pytest.mark.parametrize("wname", ["C1", "C2", "C3"])
def test_configs_full_compare(wname):
    """The small configurations, every output element against the oracle."""
    w = workloads.ATTN[wname]
    print("running", wname, w.describe(), flush=True)
    q, k, v = workloads.workload_inputs(w)
    o, lse = run_gpu(q, k, v, w.causal, w.dtype)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.causal)
    check(wname, o, lse, o_ref, lse_ref, w.dtype)


@pytest.mark.parametrize("wname", ["C4", "C5"])
def test_configs_sampled_rows(wname):
    """Full-size configurations in the launch configuration the benchmark times;
    sampled rows (first/last rows, tile edges, random rows) against the oracle,
    and every element finite."""
    w = workloads.ATTN[wname]
    print("running", wname, w.describe(), flush=True)
    q, k, v = workloads.workload_inputs(w)
    o, lse = run_gpu(q, k, v, w.causal, w.dtype)
    rows = workloads.sample_rows(w.B, w.H, w.N, 384, seed=w.seed)
    o_ref, lse_ref = oracle.attn_rows(q, k, v, w.causal, rows)
    o_rows = o.reshape(-1, w.D)[rows]
    lse_rows = lse.reshape(-1)[rows]
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    check(wname + " sampled", o_rows, lse_rows, o_ref, lse_ref, w.dtype)


LONG = [
    # (B, H, N, D, causal, dtype): a million-token causal head at D = 128 (the
    # 8-wave pipeline kernel, 4096 workgroups) and a ragged half-million-token
    # non-causal pair at D = 64 (the unit kernel, two row blocks per wave);
    # within-head offsets reach N*D = 2^27.
    (1, 1, 1 << 20, 128, True, "f16"),
    (1, 2, (1 << 19) + 37, 64, False, "bf16"),
]


@pytest.mark.parametrize("shape", LONG, ids=lambda s: "B%dH%dN%dD%d_%s_%s" % (
    s[0], s[1], s[2], s[3], "causal" if s[4] else "full", s[5]))
def test_long_sequences_sampled_rows(shape):
    """Very long sequences: sampled rows (first and last rows, tile edges,
    random rows) against the oracle, and every element finite."""
    B, H, N, D, causal, dtype = shape
    print("running long sequence", shape, flush=True)
    q, k, v = workloads.attn_inputs(B, H, N, D, dtype, seed=N % 1000 + D)
    o, lse = run_gpu(q, k, v, causal, dtype)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = workloads.sample_rows(B, H, N, 48, seed=N % 997)
    o_ref, lse_ref = oracle.attn_rows(q, k, v, causal, rows)
    check("long %s" % (shape,), o.reshape(-1, D)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, dtype)


def test_causal_prefix_is_bit_exact():
    """Changing keys/values after row i leaves rows <= i bit-identical (masked keys contribute 0)."""
    B, H, N, D = 1, 2, 700, 128
    q, k, v = workloads.attn_inputs(B, H, N, D, "f16", 77)
    print("running causal prefix B1 H2 N700 D128", flush=True)
    o1, l1 = run_gpu(q, k, v, True, "f16")
    i0 = 333
    k2, v2 = k.clone(), v.clone()
    g = torch.Generator().manual_seed(78)
    k2[:, :, i0 + 1:] = (torch.randn(k2[:, :, i0 + 1:].shape, generator=g) * 4).half()
    v2[:, :, i0 + 1:] = (torch.randn(v2[:, :, i0 + 1:].shape, generator=g) * 4).half()
    o2, l2 = run_gpu(q, k2, v2, True, "f16")
    assert np.array_equal(o1[:, :, : i0 + 1], o2[:, :, : i0 + 1])
    assert np.array_equal(l1[:, :, : i0 + 1], l2[:, :, : i0 + 1])


@pytest.mark.parametrize("shape", [(1, 1, 520, 64), (1, 512, 300, 128)],
                         ids=lambda s: "B%dH%dN%dD%d" % s)
def test_key_shift_invariance_on_gpu(shape):
    """Adding u = 2 e_5 to every key shifts each query's scores by the same
    c_i = 2 q_i[5] / sqrt(D): the softmax weights, and so O, are unchanged and
    LSE moves by exactly c_i (softmax study, section 3.3: a constant added to
    a row).  Column 5 of K is put on multiples of 2^-4 in (-8, 8), where fp16
    represents k + 2 exactly, so the shifted input is the exact shift.  The GPU
    result on the shifted keys is checked against the oracle on the original
    keys (plus c_i for LSE) at the stated tolerances.  (B1 H1 runs the 4-wave
    ring kernel, B1 H512 the 8-wave kernel.)"""
    B, H, N, D = shape
    q, k, v = workloads.attn_inputs(B, H, N, D, "f16", 79)
    k = k.clone()
    k[..., 5] = (torch.round(k[..., 5].float() * 16.0).clamp(-127, 127) / 16.0).half()
    k2 = k.clone()
    k2[..., 5] = (k[..., 5].float() + 2.0).half()
    assert torch.equal(k2[..., 5].float() - k[..., 5].float(), torch.full_like(k[..., 5].float(), 2.0))
    print("running shift invariance B%d H%d N%d D%d" % shape, flush=True)
    o2, l2 = run_gpu(q, k2, v, True, "f16")
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, True)
    c = oracle.to_f64(q)[..., 5] * 2.0 / np.sqrt(D)
    check("shift invariance B%d H%d N%d D%d" % shape, o2, l2 - c, o_ref, lse_ref, "f16")


def test_deterministic():
    """Two runs on the same inputs are bit-identical (fixed reduction order, no races)."""
    w = workloads.ATTN["C2"]
    q, k, v = workloads.workload_inputs(w)
    print("running determinism", w.describe(), flush=True)
    o1, l1 = run_gpu(q, k, v, w.causal, w.dtype)
    o2, l2 = run_gpu(q, k, v, w.causal, w.dtype)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_identical_keys_give_prefix_mean_on_gpu():
    """All keys equal: O_i is the running mean of v_0..v_i, LSE_i = s + ln(i+1)."""
    B, H, N, D = 1, 1, 300, 128
    q, _, v = workloads.attn_inputs(B, H, N, D, "bf16", 80)
    k = torch.zeros_like(q)
    print("running identical keys B1 H1 N300 D128 bf16", flush=True)
    o, lse = run_gpu(q, k, v, True, "bf16")
    vv = oracle.to_f64(v)[0, 0]
    mean = np.cumsum(vv, axis=0) / np.arange(1, N + 1)[:, None]
    assert np.abs(o[0, 0] - mean).max() <= tolerances.ATTN_O["bf16"]
    assert np.abs(lse[0, 0] - np.log(np.arange(1, N + 1))).max() <= tolerances.ATTN_LSE


# Shapes with B*H*ceil(N/256) >= 512 run 8-wave workgroups of 256 query rows
# (the tile-lagged pipeline kernel at D = 128, the key-half unit kernel at
# D = 64); the small shapes above run 4-wave workgroups.  The pipeline kernel
# runs its key tiles after the first in groups of four plus 0-3 more: the
# shapes cover every remainder, ragged key tails and several query tiles.
# Shapes on both sides of each kernel-selection boundary at D = 128: the
# key-split kernel takes B*H*ceil(N/64) <= 512, the ring kernel up to
# B*H*ceil(N/256) < 512, the pipeline kernel beyond.
BOUNDARY = [
    # (B, H, N, D, sigma_qk, kernel)
    (1, 32, 1024, 128, 1.0, "key split, 512 workgroups"),
    (1, 32, 1025, 128, 1.0, "ring, 33 64-row tiles per head"),
    (2, 7, 2300, 128, 3.0, "key split, large logits, 504 workgroups"),
    (1, 16, 2100, 128, 3.0, "ring, large logits, 528 64-row tiles"),
    (1, 1, 32768, 128, 1.0, "key split, one head, 512 workgroups"),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", BOUNDARY, ids=lambda s: "B%dH%dN%dD%d" % s[:4])
def test_selection_boundaries_match_oracle(shape, causal, dtype):
    B, H, N, D, sigma, _ = shape
    seed = 2500 + N * 3 + B + (1 if causal else 0)
    q, k, v = workloads.attn_inputs(B, H, N, D, dtype, seed, sigma_qk=sigma)
    name = "boundary attn %s %s B%d H%d N%d D%d sigma %g seed %d" % (
        "causal" if causal else "full", dtype, B, H, N, D, sigma, seed)
    print("running", name, flush=True)
    o, lse = run_gpu(q, k, v, causal, dtype)
    if N > 4096:
        # one head of 32768 rows: rows near the head's ends and tile edges, and
        # a seeded spread through it (flat row ids; B = H = 1)
        g = torch.Generator().manual_seed(seed)
        rows = sorted({0, 1, 63, 64, N - 1} | set(torch.randint(0, N, (120,), generator=g).tolist()))
        o_ref, lse_ref = oracle.attn_rows(q, k, v, causal, rows)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        check(name, o.reshape(-1, D)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, dtype)
    else:
        o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal)
        check(name, o, lse, o_ref, lse_ref, dtype)


WIDE = [
    # (B, H, N, D, sigma_qk)
    (1, 512, 64, 128, 1.0),     # one 64-key tile per head
    (1, 512, 200, 64, 1.5),     # one partial query tile per head
    (2, 128, 300, 128, 3.0),    # ragged second tile; large logits
    (1, 256, 513, 64, 3.0),     # one row past a 256-row tile edge
    (1, 256, 350, 128, 2.0),    # 6 key tiles (ragged): remainder 1
    (1, 256, 400, 128, 1.5),    # 7 key tiles (ragged): remainder 2
    (1, 128, 1024, 128, 1.0),   # 4 query tiles, 16 key tiles: remainder 3
    (1, 96, 1500, 128, 1.0),    # 6 query tiles, ragged 24th key tile
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", WIDE, ids=lambda s: "B%dH%dN%dD%ds%g" % s)
def test_wide_shapes_match_oracle(shape, causal, dtype):
    B, H, N, D, sigma = shape
    assert B * H * ((N + 255) // 256) >= 512
    seed = 2000 + N * 7 + D + (1 if causal else 0)
    q, k, v = workloads.attn_inputs(B, H, N, D, dtype, seed, sigma_qk=sigma)
    name = "wide attn %s %s B%d H%d N%d D%d sigma %g seed %d" % (
        "causal" if causal else "full", dtype, B, H, N, D, sigma, seed)
    print("running", name, flush=True)
    o, lse = run_gpu(q, k, v, causal, dtype)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal)
    check(name, o, lse, o_ref, lse_ref, dtype)


# Causal grids of the 4-wave kernel (128-row workgroups, two per CU) that are
# resident in one round and larger than the CU count: 256 < B*H*ceil(N/128)
# <= 512 with B*H*ceil(N/256) < 512.  Their order is folded (the second half
# of the grid shortest first); an odd number of query tiles splits unevenly.
FOLDED = [
    # (B, H, N, D)
    (1, 40, 1152, 128),     # 9 query tiles (odd), 360 workgroups
    (2, 12, 1500, 64),      # 12 query tiles, ragged last tile, 288 workgroups
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", FOLDED, ids=lambda s: "B%dH%dN%dD%d" % s)
def test_folded_one_round_grid_matches_oracle(shape, dtype):
    B, H, N, D = shape
    wgs = B * H * ((N + 127) // 128)
    assert 256 < wgs <= 512 and B * H * ((N + 255) // 256) < 512
    seed = 3000 + N + D
    q, k, v = workloads.attn_inputs(B, H, N, D, dtype, seed, sigma_qk=1.5)
    name = "folded grid attn causal %s B%d H%d N%d D%d seed %d" % (dtype, B, H, N, D, seed)
    print("running", name, flush=True)
    o, lse = run_gpu(q, k, v, True, dtype)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, True)
    check(name, o, lse, o_ref, lse_ref, dtype)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_wide_ramped_logits(causal, dtype, D):
    """Scores that rise (or fall) steeply along the keys: with q near 1 and
    k_j near slope_h * j, every key half of a rising head holds a new row
    maximum far above the previous one, so the reference maximum has to move
    for every half; falling heads never move it after the first key; flat and
    noisy heads sit in between.  Scaled logits reach several hundred."""
    B, H, N = 1, 512, 256
    g = torch.Generator().manual_seed(2301 + D)
    slopes = torch.tensor([0.05, -0.05, 0.3, 0.0, 0.02, -0.3, 0.15, 0.01])
    slope = slopes[torch.arange(H) % len(slopes)].view(1, H, 1, 1)
    j = torch.arange(N, dtype=torch.float32).view(1, 1, N, 1)
    td = workloads.TORCH_DTYPE[dtype]
    q = (1.0 + 0.1 * torch.randn((B, H, N, D), generator=g)).to(td).contiguous()
    k = (slope * j + 0.5 * torch.randn((B, H, N, D), generator=g)).to(td).contiguous()
    v = torch.randn((B, H, N, D), generator=g).to(td).contiguous()
    name = "wide ramped logits %s %s B1 H512 N256 D%d" % ("causal" if causal else "full", dtype, D)
    print("running", name, flush=True)
    o, lse = run_gpu(q, k, v, causal, dtype)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal)
    assert np.abs(lse_ref).max() > 300.0
    check(name, o, lse, o_ref, lse_ref, dtype)
