"""Pins of the FP64 attention-backward oracle (CPU only).

The pages give no backward algorithm (the FA page, section 7, only says the
log-sum-exp is kept for it), so the oracle is the calculus of the forward
definition.  It is checked against: torch float64 autograd through an
explicit softmax; central finite differences of the (separately pinned)
forward oracle; exact identities (keys' dK sum to zero, dV sums to the sum of
dO, a single key gives dQ = dK = 0 and dV = dO, identical keys give dQ = 0);
and the causal dependency structure, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle


def rand(*shape, scale=1.0, seed=0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64) * scale


def autograd_ref(q, k, v, do, causal):
    qq, kk, vv = [x.clone().requires_grad_() for x in (q, k, v)]
    N, D = q.shape[-2], q.shape[-1]
    s = qq @ kk.transpose(-1, -2) / np.sqrt(D)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, -1) @ vv
    (o * do).sum().backward()
    return qq.grad.numpy(), kk.grad.numpy(), vv.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 2, 9, 8), (2, 1, 33, 16), (1, 1, 70, 64)])
def test_matches_torch_autograd_float64(shape, causal):
    q, k, v, do = (rand(*shape, scale=1.5, seed=s) for s in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal)
    rq, rk, rv = autograd_ref(q, k, v, do, causal)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_central_differences_of_the_forward_oracle(causal):
    """dL/dx for L = sum(O * dO), O from oracle.attn_fwd, by central differences."""
    shape = (1, 1, 7, 4)
    q, k, v, do = (rand(*shape, seed=10 + s).numpy() for s in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal)
    loss = lambda q_, k_, v_: float((oracle.attn_fwd(q_, k_, v_, causal)[0] * do).sum())
    eps = 1e-5
    rng = np.random.default_rng(1)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(6):
            idx = (0, 0, int(rng.integers(7)), int(rng.integers(4)))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            dn = loss(*args)
            assert abs((up - dn) / (2 * eps) - grad[idx]) < 1e-8, (which, idx)


@pytest.mark.parametrize("causal", [True, False])
def test_key_gradients_sum_to_zero_and_dv_to_the_dout_sum(causal):
    """Each softmax row sums to 1, so sum_j dS_ij = 0 (hence sum_j dK_j = 0)
    and sum_j P_ij = 1 (hence sum_j dV_j = sum_i dO_i)."""
    q, k, v, do = (rand(2, 3, 40, 16, scale=2.0, seed=20 + s) for s in range(4))
    _, dk, dv = oracle.attn_bwd(q, k, v, do, causal)
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    np.testing.assert_allclose(dv.sum(axis=2), do.numpy().sum(axis=2), rtol=0, atol=1e-12)


def test_single_key_and_identical_keys():
    q, k, v, do = (rand(1, 2, 1, 8, seed=30 + s) for s in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, True)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_array_equal(dv, do.numpy())
    q, v, do = (rand(1, 1, 25, 8, seed=40 + s) for s in range(3))
    k = rand(1, 1, 1, 8, seed=43).expand(1, 1, 25, 8).contiguous()
    for causal in (True, False):
        dq, _, _ = oracle.attn_bwd(q, k, v, do, causal)
        assert np.abs(dq).max() < 1e-13


def test_causal_dependency_structure_is_exact():
    """Causal: dK_j, dV_j read only rows i >= j; dQ_i reads only keys j <= i."""
    q, k, v, do = (rand(1, 1, 30, 16, seed=50 + s) for s in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, True)
    j = 12
    q2, do2 = q.clone(), do.clone()
    q2[..., :j, :] += 1.0
    do2[..., :j, :] -= 0.5
    _, dk2, dv2 = oracle.attn_bwd(q2, k, v, do2, True)
    assert np.array_equal(dk[..., j:, :], dk2[..., j:, :])
    assert np.array_equal(dv[..., j:, :], dv2[..., j:, :])
    k3, v3 = k.clone(), v.clone()
    k3[..., j + 1:, :] *= 3.0
    v3[..., j + 1:, :] += 2.0
    dq3, _, _ = oracle.attn_bwd(q, k3, v3, do, True)
    assert np.array_equal(dq[..., :j + 1, :], dq3[..., :j + 1, :])


def test_selected_heads_equal_the_full_result():
    q, k, v, do = (rand(2, 3, 20, 8, seed=60 + s) for s in range(4))
    full = oracle.attn_bwd(q, k, v, do, True)
    part = oracle.attn_bwd(q, k, v, do, True, heads=[4, 1])
    for f, p in zip(full, part):
        assert np.array_equal(f.reshape(6, 20, 8)[[4, 1]], p)


# ------------------------------------------------- grouped K/V heads (GQA)

def autograd_gqa(q, k, v, do, causal):
    """torch float64 autograd through repeat_interleave of the K/V heads."""
    qq, kk, vv = [x.clone().requires_grad_() for x in (q, k, v)]
    g = q.shape[1] // k.shape[1]
    kr = torch.repeat_interleave(kk, g, dim=1)
    vr = torch.repeat_interleave(vv, g, dim=1)
    N, D = q.shape[-2], q.shape[-1]
    s = qq @ kr.transpose(-1, -2) / np.sqrt(D)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, -1) @ vr
    (o * do).sum().backward()
    return qq.grad.numpy(), kk.grad.numpy(), vv.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 4, 2, 17, 8), (2, 6, 3, 33, 16), (1, 8, 1, 40, 32)])
def test_gqa_matches_torch_autograd_float64(shape, causal):
    B, H, Hkv, N, D = shape
    q = rand(B, H, N, D, scale=1.5, seed=70)
    k = rand(B, Hkv, N, D, scale=1.5, seed=71)
    v = rand(B, Hkv, N, D, seed=72)
    do = rand(B, H, N, D, seed=73)
    dq, dk, dv = oracle.attn_bwd_gqa(q, k, v, do, causal)
    assert dk.shape == (B, Hkv, N, D) and dq.shape == (B, H, N, D)
    rq, rk, rv = autograd_gqa(q, k, v, do, causal)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_gqa_with_one_head_per_group_is_the_plain_backward():
    q, k, v, do = (rand(2, 3, 21, 16, seed=80 + s) for s in range(4))
    for causal in (True, False):
        a = oracle.attn_bwd_gqa(q, k, v, do, causal)
        b = oracle.attn_bwd(q, k, v, do, causal)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_gqa_group_sums_and_invariants():
    """dK of a shared head is the sum of the group's per-head dK against that
    head (so its keys still sum to zero); dV of a shared head sums to the sum
    of the group's dO."""
    B, H, Hkv, N, D = 1, 6, 2, 25, 8
    q, do = rand(B, H, N, D, seed=90), rand(B, H, N, D, seed=91)
    k, v = rand(B, Hkv, N, D, scale=2.0, seed=92), rand(B, Hkv, N, D, seed=93)
    dq, dk, dv = oracle.attn_bwd_gqa(q, k, v, do, True)
    g = H // Hkv
    for j in range(Hkv):
        acc_k = np.zeros((N, D))
        acc_v = np.zeros((N, D))
        for h in range(j * g, (j + 1) * g):
            dqh, dkh, dvh = oracle.attn_bwd(q[:, h:h + 1], k[:, j:j + 1], v[:, j:j + 1],
                                            do[:, h:h + 1], True)
            assert np.array_equal(dqh[0, 0], dq[0, h])
            acc_k += dkh[0, 0]
            acc_v += dvh[0, 0]
        np.testing.assert_allclose(dk[0, j], acc_k, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv[0, j], acc_v, rtol=0, atol=1e-13)
        assert np.abs(dk[0, j].sum(axis=0)).max() < 1e-12
        np.testing.assert_allclose(dv[0, j].sum(axis=0), do[0, j * g:(j + 1) * g].numpy().sum(axis=(0, 1)),
                                   rtol=0, atol=1e-12)


def test_gqa_selected_kv_heads_equal_the_full_result():
    B, H, Hkv, N, D = 2, 4, 2, 19, 8
    q, do = rand(B, H, N, D, seed=100), rand(B, H, N, D, seed=101)
    k, v = rand(B, Hkv, N, D, seed=102), rand(B, Hkv, N, D, seed=103)
    dq, dk, dv = oracle.attn_bwd_gqa(q, k, v, do, True)
    pq, pk, pv = oracle.attn_bwd_gqa(q, k, v, do, True, kv_heads=[3, 0])
    assert np.array_equal(pk, dk.reshape(4, N, D)[[3, 0]])
    assert np.array_equal(pv, dv.reshape(4, N, D)[[3, 0]])
    assert np.array_equal(pq, dq.reshape(8, N, D)[[6, 7, 0, 1]])
