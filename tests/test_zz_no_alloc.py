"""paged_decode_noalloc: paged decode with the segment states in the
library's fixed per-device array instead of a caller workspace.

GPU: two calls in a row (the second on a smaller problem, so the array still
holds the first call's states), each compared bit for bit with paged_decode on
a NaN-filled workspace and, within the attention tolerances, with the FP64
oracle.  CPU: the size limit and the argument checks reject before any HIP
call.
"""
import re

import numpy as np
import pytest
import torch

import oracle
import online_softmax_causal_amd as osc
import workloads
from tests import tolerances
from tests.test_abi import BASE, MB, ROOT
from tests.test_gpu_attn import dev

PAGED_MAX = 4096  # PAGED_MAX_SPLITS


def header_scratch_bytes():
    text = open(ROOT + "/include/osc_attn.h").read()
    m = re.search(r"#define\s+PAGED_NOALLOC_SCRATCH_BYTES\s+\((\d+) \* 1024 \* 1024\)", text)
    assert m
    return int(m.group(1)) << 20


def test_binding_limit_matches_header():
    assert osc.PAGED_NOALLOC_SCRATCH_BYTES == header_scratch_bytes()


def call_noalloc(B, Hq, Hkv, D, T, P, max_pages, splits, q=BASE):
    lib = osc.load()
    cache = BASE + 256 * MB
    bt = BASE + (1 << 36)
    ln = bt + 64 * MB
    o = ln + 64 * MB
    lse = o + (1 << 34)
    return lib.paged_decode_noalloc(q, cache, bt, ln, o, lse, B, Hq, Hkv, D, T, P, max_pages, 0,
                                    splits, None)


def test_rejects_states_beyond_the_array_before_any_hip_call():
    # 4096 requests x 32 heads x 16 segments x 130 words x 4 bytes > 32 MiB
    B, Hq, Hkv, D, T, max_pages = 4096, 32, 8, 128, 16, 2048
    need = osc.paged_decode_workspace(B, Hq, Hkv, D, T, max_pages, 16)
    assert need > osc.PAGED_NOALLOC_SCRATCH_BYTES
    assert call_noalloc(B, Hq, Hkv, D, T, 1, max_pages, 16) == 7      # ATTN_ERR_WORKSPACE


def test_rejects_bad_arguments_like_paged_decode():
    assert call_noalloc(2, 8, 2, 128, 16, 4, 2, 0, q=None) == 1        # ATTN_ERR_NULL
    assert call_noalloc(2, 8, 3, 128, 16, 4, 2, 0) == 2                # Hq % Hkv != 0
    assert call_noalloc(2, 8, 2, 96, 16, 4, 2, 0) == 3                 # D = 96
    assert call_noalloc(2, 8, 2, 128, 16, 4, 2, 0, q=BASE + 2) == 4    # misaligned q
    assert call_noalloc(2, 8, 2, 128, 16, 4, 2, PAGED_MAX + 1) == 2


def run_pair(B, Hq, Hkv, D, T, lens, splits, dtype, seed):
    d = dev()
    max_pages = (max(lens) + T - 1) // T + 1
    P = B * max_pages + 3
    q, cache, bt, ln = workloads.decode_inputs(B, Hq, Hkv, D, T, P, max_pages, lens, dtype, seed,
                                               sigma_qk=1.5)
    qd, cd = q.to(d), cache.to(d)
    btd, lnd = bt.to(d), ln.to(d)
    need = osc.paged_decode_workspace(B, Hq, Hkv, D, T, max_pages, splits)
    assert 0 <= need <= osc.PAGED_NOALLOC_SCRATCH_BYTES
    ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device=d)
    outs = []
    for with_ws in (True, False):
        o = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=d)
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=d)
        if with_ws:
            osc.paged_decode(qd, cd, btd, lnd, o, lse, B, Hq, Hkv, D, T, P, max_pages, dtype,
                             splits, ws, ws.numel() * 4)
        else:
            osc.paged_decode_noalloc(qd, cd, btd, lnd, o, lse, B, Hq, Hkv, D, T, P, max_pages,
                                     dtype, splits)
        torch.cuda.synchronize()
        outs.append((o.cpu().double().numpy(), lse.cpu().double().numpy()))
    (o_ws, l_ws), (o_na, l_na) = outs
    assert np.isfinite(o_na).all() and np.isfinite(l_na).all()
    assert np.array_equal(o_na, o_ws) and np.array_equal(l_na, l_ws)
    o_ref, l_ref = oracle.paged_decode(q, cache, bt.numpy(), ln.numpy(), T)
    eo = np.abs(o_na.reshape(-1, D) - o_ref).max()
    el = np.abs(l_na.reshape(-1) - l_ref).max()
    print("noalloc %s B%d Hq%d Hkv%d D%d T%d need %d: max|dO| %.3e max|dLSE| %.3e" % (
        dtype, B, Hq, Hkv, D, T, need, eo, el), flush=True)
    assert eo <= tolerances.ATTN_O[dtype] and el <= tolerances.ATTN_LSE
    return need


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_noalloc_matches_paged_decode_twice_second_smaller(dtype):
    print("running noalloc pair %s" % dtype, flush=True)
    n1 = run_pair(8, 32, 8, 128, 16, (4096, 3000, 1, 33, 2047, 2048, 2049, 777), 0, dtype, 7201)
    n2 = run_pair(3, 8, 2, 64, 8, (300, 1, 95), 5, dtype, 7202)
    assert 0 < n2 < n1
    # one segment: no states at all
    assert run_pair(2, 4, 4, 128, 16, (40, 17), 1, dtype, 7203) == 0
