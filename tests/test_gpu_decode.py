"""GPU parity of paged_decode (through the C ABI) against the FP64 oracle.

Outputs and workspace are NaN-prefilled, so an unwritten element or a merge
that reads a segment the kernel did not write fails.  Tolerances as for
attention: max-abs O 4e-3 (fp16) / 1.6e-2 (bf16), LSE 1e-3.
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


def run_decode(q, cache, bt, lens, page_size, dtype, splits=0, ws=None):
    d = dev()
    B, Hq, D = q.shape
    P, _, T, Hkv, _ = cache.shape
    max_pages = bt.shape[1]
    need = osc.paged_decode_workspace(B, Hq, Hkv, D, page_size, max_pages, splits)
    assert need >= 0
    if ws is None:
        ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device=d)
    else:
        ws.fill_(float("nan"))
    assert ws.numel() * 4 >= need
    o = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=d)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=d)
    qd, cd = q.to(d), cache.to(d)
    btd = torch.as_tensor(np.asarray(bt), dtype=torch.int32).to(d)
    lnd = torch.as_tensor(np.asarray(lens), dtype=torch.int32).to(d)
    osc.paged_decode(qd, cd, btd, lnd, o, lse, B, Hq, Hkv, D, page_size, P, max_pages, dtype,
                     splits, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy(), need


def check(name, o, lse, o_ref, lse_ref, dtype):
    assert np.isfinite(o).all(), "%s: non-finite O" % name
    assert np.isfinite(lse).all(), "%s: non-finite LSE" % name
    eo = np.abs(o - o_ref).max()
    el = np.abs(lse - lse_ref).max()
    print("%s: max|dO| %.3e  max|dLSE| %.3e" % (name, eo, el), flush=True)
    assert eo <= tolerances.ATTN_O[dtype], "%s: O error %.3e" % (name, eo)
    assert el <= tolerances.ATTN_LSE, "%s: LSE error %.3e" % (name, el)


CASES = [
    # (B, Hq, Hkv, D, T, lengths, splits): single tokens, tile edges (31, 32,
    # 33, 64), ragged lengths, page sizes 1..64, groups of 1, 4, 8 and 32
    # heads, automatic and requested splits
    (3, 8, 2, 128, 16, (1, 31, 33), 0),
    (2, 32, 8, 128, 16, (100, 257), 0),
    (4, 4, 4, 64, 4, (32, 64, 65, 7), 0),
    (2, 32, 1, 64, 1, (70, 3), 0),
    (1, 8, 1, 128, 64, (1000,), 3),
    (2, 16, 2, 128, 8, (513, 2048), 1),
    (5, 6, 3, 64, 32, (1, 2, 600, 95, 2500), 7),
    (1, 2, 2, 128, 2, (4097,), 0),
    # large pages: 1024 tokens, and the largest page size, 65536 tokens, with
    # a request of two full pages and one that ends one token into a page
    (2, 8, 2, 64, 1024, (3000, 1025), 0),
    (2, 4, 1, 64, 65536, (131072, 65537), 0),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dHq%dHkv%dD%dT%d-%s-s%d" % (
    c[0], c[1], c[2], c[3], c[4], "_".join(map(str, c[5])), c[6]))
def test_small_cases_match_oracle(case, dtype):
    B, Hq, Hkv, D, T, lens, splits = case
    max_pages = (max(lens) + T - 1) // T + 1
    P = B * max_pages + 3
    seed = 7000 + sum(lens) + D + T
    q, cache, bt, ln = workloads.decode_inputs(B, Hq, Hkv, D, T, P, max_pages, lens, dtype, seed,
                                               sigma_qk=1.5)
    name = "decode %s B%d Hq%d Hkv%d D%d T%d lens %s splits %d seed %d" % (
        dtype, B, Hq, Hkv, D, T, lens, splits, seed)
    print("running", name, flush=True)
    o, lse, _ = run_decode(q, cache, bt, ln, T, dtype, splits)
    o_ref, lse_ref = oracle.paged_decode(q, cache, bt.numpy(), ln.numpy(), T)
    check(name, o.reshape(-1, D), lse.reshape(-1), o_ref, lse_ref, dtype)


def test_large_logits_need_the_running_max():
    """Q, K ~ N(0, 3^2): scaled logits reach |s| ~ 30 and the maximum moves."""
    lens = (3000, 1234)
    q, cache, bt, ln = workloads.decode_inputs(2, 8, 2, 128, 16, 300, 190, lens, "bf16", 7101,
                                               sigma_qk=3.0)
    print("running decode large logits", flush=True)
    o, lse, need = run_decode(q, cache, bt, ln, 16, "bf16", 0)
    assert need > 0
    o_ref, lse_ref = oracle.paged_decode(q, cache, bt.numpy(), ln.numpy(), 16)
    check("decode large logits", o.reshape(-1, 128), lse.reshape(-1), o_ref, lse_ref, "bf16")


def test_invalid_device_data_gives_nan_rows_only():
    """A length of 0, a length past the table and a used page id out of range
    poison only their own requests (and nothing is read out of range); a bad
    page id past a request's length is never looked at."""
    B, Hq, Hkv, D, T = 6, 8, 2, 128, 16
    lens = [40, 0, 300, 50, 999999, 17]
    max_pages = 20
    P = 100
    q, cache, bt, ln = workloads.decode_inputs(B, Hq, Hkv, D, T, P, max_pages, [1] * B, "f16",
                                               7102)
    bt = bt.clone()
    ln = torch.as_tensor(lens, dtype=torch.int32)
    bt[2, 5] = P + 1000      # used by request 2 (tokens 80..95)
    bt[3, 10] = -5           # past request 3's length: ignored
    bt[5, 0] = -1            # request 5's only page
    for splits in (0, 1):
        print("running decode invalid data splits %d" % splits, flush=True)
        o, lse, _ = run_decode(q, cache, bt, ln, T, "f16", splits)
        for b in (1, 2, 4, 5):
            assert np.isnan(o[b]).all() and np.isnan(lse[b]).all(), (b, splits)
        good = [0, 3]
        o_ref, lse_ref = oracle.paged_decode(q[good], cache, bt[good].numpy(), ln[good].numpy(), T)
        check("decode valid requests beside invalid ones", o[good].reshape(-1, D),
              lse[good].reshape(-1), o_ref, lse_ref, "f16")


def test_workspace_reused_second_call_smaller():
    d = dev()
    need = osc.paged_decode_workspace(4, 32, 8, 128, 16, 128, 0)
    ws = torch.empty((need // 4,), dtype=torch.float32, device=d)
    for (B, ctx, seed) in [(4, 2000, 7103), (2, 700, 7104)]:
        max_pages = (ctx + 15) // 16
        q, cache, bt, ln = workloads.decode_inputs(B, 32, 8, 128, 16, B * max_pages, max_pages,
                                                   [ctx, ctx - 5, 1, 33][:B], "f16", seed)
        print("running decode reuse B%d ctx %d" % (B, ctx), flush=True)
        o, lse, n2 = run_decode(q, cache, bt, ln, 16, "f16", 0, ws=ws)
        assert n2 <= need
        o_ref, lse_ref = oracle.paged_decode(q, cache, bt.numpy(), ln.numpy(), 16)
        check("decode reuse B%d" % B, o.reshape(-1, 128), lse.reshape(-1), o_ref, lse_ref, "f16")


def test_deterministic_and_split_consistent():
    q, cache, bt, ln = workloads.decode_inputs(2, 16, 4, 128, 16, 300, 128, (2040, 1777), "f16",
                                               7105)
    print("running decode determinism", flush=True)
    o1, l1, _ = run_decode(q, cache, bt, ln, 16, "f16", 0)
    o2, l2, _ = run_decode(q, cache, bt, ln, 16, "f16", 0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3, need1 = run_decode(q, cache, bt, ln, 16, "f16", 1)
    assert need1 == 0
    # one segment against many: both within tolerance of each other
    assert np.abs(o1 - o3).max() <= tolerances.ATTN_O["f16"]
    assert np.abs(l1 - l3).max() <= tolerances.ATTN_LSE


# Segments of at most 512 tokens run the decode kernel's VGPR-form build, longer
# ones the other build.  With 16-token pages and 64 pages per request (1024
# tokens of capacity, 32 tiles of 32) the requested splits give segments of
# 256 and 512 tokens (short build) and 1024 (long build, one segment); with 69
# pages (1104 tokens, 35 tiles) two splits give 576-token segments (long build,
# two segments).  Every plan against the oracle.
@pytest.mark.parametrize("lens,splits", [((1008, 700), 4), ((1008, 700), 2), ((1008, 700), 1),
                                         ((1080, 999), 2)],
                         ids=["seg256", "seg512", "seg1024", "seg576"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_both_decode_builds_around_the_segment_boundary(lens, splits, dtype):
    B, Hq, Hkv, D, T = 2, 16, 4, 128, 16
    max_pages = (max(lens) + T - 1) // T + 1
    P = B * max_pages + 3
    seed = 7300 + sum(lens)
    q, cache, bt, ln = workloads.decode_inputs(B, Hq, Hkv, D, T, P, max_pages, lens, dtype, seed,
                                               sigma_qk=1.5)
    name = "decode boundary %s lens %s splits %d seed %d" % (dtype, lens, splits, seed)
    print("running", name, flush=True)
    o, lse, _ = run_decode(q, cache, bt, ln, T, dtype, splits)
    o_ref, lse_ref = oracle.paged_decode(q, cache, bt.numpy(), ln.numpy(), T)
    check(name, o.reshape(-1, D), lse.reshape(-1), o_ref, lse_ref, dtype)


@pytest.mark.parametrize("name", ["D1", "D32"])
def test_benchmark_workload_sampled(name):
    """The benchmark's shapes (B8 Hq32 Hkv8 D128 page 16) in its launch
    configuration (automatic split), checked on sampled (request, head) pairs."""
    w = workloads.DECODE[name]
    print("running", w.describe(), flush=True)
    q, cache, bt, ln = workloads.decode_workload_inputs(w)
    o, lse, need = run_decode(q, cache, bt, ln, w.page_size, w.dtype, 0)
    assert need > 0
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    g = torch.Generator().manual_seed(w.seed)
    rows = sorted({0, w.B * w.Hq - 1} | set(torch.randint(0, w.B * w.Hq, (30,), generator=g).tolist()))
    o_ref, lse_ref = oracle.paged_decode(q, cache, bt.numpy(), ln.numpy(), w.page_size, rows=rows)
    check(w.describe(), o.reshape(-1, w.D)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, w.dtype)
