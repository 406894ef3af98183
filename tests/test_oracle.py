"""Pins for the FP64 oracle (CPU only).

Each test checks the oracle against something other than itself: a closed
form, an invariant of the definition, brute force on a tiny exact case, or an
independent library routine.  The cases are chosen so that a plausible slip
in the oracle (dropped or wrong scale, transposed operand, K used in place of
V, an off-by-one causal mask, log2 instead of ln in the LSE, a missing
max-subtraction, rows mixed across heads) fails at least one of them.

Definitions: attention per "CUDA FlashAttention: from online softmax to
long-sequence IO limits" (chengzipai.xyz) sections 1, 3 and 4; row softmax per
the softmax kernel study (lpnh.cn/news/2830604) sections 3.1-3.3.
"""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(1234)


def rand(*shape, scale=1.0, rng=RNG):
    return rng.standard_normal(shape) * scale


# ------------------------------------------------------------------ stage 1

@pytest.mark.parametrize("D", [4, 16, 64])
def test_stage1_picks_one_key_column(D):
    """One-hot query rows: s_ij = c * K[j, a_i] / sqrt(D) exactly.

    Integer K and c make the dot product exact and sqrt(D) is a power of two,
    so equality is exact.  A transposed operand, a wrong row or column index
    or a missing / wrong scale changes the result.
    """
    N = 9
    k = RNG.integers(-8, 9, size=(N, D)).astype(np.float64)
    a = RNG.integers(0, D, size=N)
    c = RNG.integers(1, 6, size=N).astype(np.float64)
    q = np.zeros((N, D))
    q[np.arange(N), a] = c
    for causal in (True, False):
        for i in range(N):
            s = oracle.attn_scores(q, k, causal, i)
            nkeys = i + 1 if causal else N
            assert s.shape == (nkeys,)
            expect = c[i] * k[:nkeys, a[i]] / math.sqrt(D)
            assert np.array_equal(s, expect)


def test_stage1_causal_key_count_and_prefix():
    """Causal row i sees keys 0..i (j <= i, FA page section 1); non-causal sees all N."""
    N, D = 7, 8
    q, k = rand(N, D), rand(N, D)
    full = [oracle.attn_scores(q, k, False, i) for i in range(N)]
    for i in range(N):
        s = oracle.attn_scores(q, k, True, i)
        assert s.shape == (i + 1,)
        assert np.array_equal(s, full[i][: i + 1])


# --------------------------------------------------------- whole attention

@pytest.mark.parametrize("D", [4, 64, 128])
def test_single_key_returns_v0(D):
    """N = 1: the only weight is 1, so O = v_0 exactly and lse = q0.k0/sqrt(D)."""
    q = RNG.integers(-4, 5, size=(1, 2, 1, D)).astype(np.float64)
    k = RNG.integers(-4, 5, size=(1, 2, 1, D)).astype(np.float64)
    v = rand(1, 2, 1, D)
    for causal in (True, False):
        o, lse = oracle.attn_fwd(q, k, v, causal)
        assert np.array_equal(o, v)
        for h in range(2):
            dot = sum(int(x) * int(y) for x, y in zip(q[0, h, 0], k[0, h, 0]))
            assert lse[0, h, 0] == pytest.approx(dot / math.sqrt(D), rel=0, abs=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_identical_keys_give_prefix_mean(causal):
    """All keys equal to u: every weight in row i is 1/|J_i|.

    O_i is the mean of v_0..v_i (causal) or of all rows (non-causal), and
    lse_i = q_i.u/sqrt(D) + ln|J_i|.  u is a multiple of a basis vector so
    q_i.u is a single product.
    """
    N, D = 11, 16
    q = rand(1, 1, N, D)
    u = np.zeros(D)
    u[3] = 2.5
    k = np.broadcast_to(u, (1, 1, N, D)).copy()
    v = rand(1, 1, N, D)
    o, lse = oracle.attn_fwd(q, k, v, causal)
    for i in range(N):
        n = i + 1 if causal else N
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), rtol=0, atol=1e-13)
        expect = q[0, 0, i, 3] * 2.5 / 4.0 + math.log(n)
        assert lse[0, 0, i] == pytest.approx(expect, abs=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_zero_queries_give_uniform_weights(causal):
    """Q = 0: all logits are 0, weights are uniform, lse_i = ln|J_i|."""
    B, H, N, D = 2, 3, 10, 8
    q = np.zeros((B, H, N, D))
    k, v = rand(B, H, N, D, scale=5.0), rand(B, H, N, D)
    o, lse = oracle.attn_fwd(q, k, v, causal)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                n = i + 1 if causal else N
                np.testing.assert_allclose(o[b, h, i], v[b, h, :n].mean(axis=0), atol=1e-13)
                assert lse[b, h, i] == pytest.approx(math.log(n), abs=1e-14)


@pytest.mark.parametrize("a", [-30.0, -2.0, 0.5, 7.0, 40.0])
def test_two_keys_logistic(a):
    """Row 1 over keys {0,1} with s_10 = a, s_11 = 0: p_0 = 1/(1+e^-a) (the logistic).

    Also lse_1 = ln(1 + e^a).  Large |a| checks the max subtraction (no
    overflow at a = 40, where e^a alone would still be finite but e^(a*25)
    would not) and the ordering of the two weights.
    """
    D = 16
    q = np.zeros((1, 1, 2, D))
    k = np.zeros((1, 1, 2, D))
    q[0, 0, 1, 0] = a * 4.0       # s = a*4*1/sqrt(16) = a
    k[0, 0, 0, 0] = 1.0
    v = rand(1, 1, 2, D)
    o, lse = oracle.attn_fwd(q, k, v, True)
    p0 = 1.0 / (1.0 + math.exp(-a))
    np.testing.assert_allclose(o[0, 0, 1], p0 * v[0, 0, 0] + (1 - p0) * v[0, 0, 1],
                               rtol=1e-13, atol=1e-14)
    expect_lse = max(a, 0.0) + math.log1p(math.exp(-abs(a)))
    assert lse[0, 0, 1] == pytest.approx(expect_lse, abs=1e-13)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])


def test_large_logits_stay_finite():
    """Logits of 750 overflow exp (double) unless the row max is subtracted first
    (FA page section 2: without subtracting the row maximum, exp overflows)."""
    D = 4
    q = np.zeros((1, 1, 3, D))
    k = np.zeros((1, 1, 3, D))
    q[0, 0, :, 0] = 1500.0     # s = 750 * k[:,0]
    k[0, 0, :, 0] = [1.0, 1.0, 0.999]
    v = rand(1, 1, 3, D)
    o, lse = oracle.attn_fwd(q, k, v, False)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    w = np.exp(np.array([0.0, 0.0, -0.75]))
    w /= w.sum()
    np.testing.assert_allclose(o[0, 0, 0], w @ v[0, 0], rtol=1e-12)
    assert lse[0, 0, 0] == pytest.approx(750.0 + math.log(2 + math.exp(-0.75)), abs=1e-12)
    y = oracle.row_softmax(np.array([[800.0, 799.0]]))
    np.testing.assert_allclose(y[0], [1 / (1 + math.exp(-1.0)), 1 / (1 + math.exp(1.0))],
                               rtol=1e-15)


@pytest.mark.parametrize("causal", [True, False])
def test_key_shift_invariance(causal):
    """K' = K + 1 u^T adds q_i.u/sqrt(D) to every logit of row i.

    O is unchanged and lse shifts by exactly that amount (softmax shift
    invariance, softmax study section 3.3: a constant added to a whole row).
    u = c * e_2, so q_i.u = c * q_i[2].
    """
    B, H, N, D = 1, 2, 13, 64
    q, k, v = rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    k2 = k.copy()
    k2[..., 2] += 3.0
    o, lse = oracle.attn_fwd(q, k, v, causal)
    o2, lse2 = oracle.attn_fwd(q, k2, v, causal)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2 - lse, q[..., 2] * 3.0 / 8.0, rtol=0, atol=1e-12)


def test_causal_prefix_property():
    """Row i depends only on keys/values 0..i: perturbing later rows leaves it bit-identical."""
    B, H, N, D = 1, 2, 16, 8
    q, k, v = rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    o, lse = oracle.attn_fwd(q, k, v, True)
    i0 = 6
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i0 + 1:] = rand(B, H, N - i0 - 1, D, scale=10.0)
    v2[:, :, i0 + 1:] = rand(B, H, N - i0 - 1, D, scale=10.0)
    o2, lse2 = oracle.attn_fwd(q, k2, v2, True)
    assert np.array_equal(o2[:, :, : i0 + 1], o[:, :, : i0 + 1])
    assert np.array_equal(lse2[:, :, : i0 + 1], lse[:, :, : i0 + 1])
    assert not np.allclose(o2[:, :, i0 + 1:], o[:, :, i0 + 1:])


def test_noncausal_permutations():
    """Non-causal: permuting (K,V) rows together keeps O; permuting Q rows permutes O."""
    B, H, N, D = 1, 1, 12, 16
    q, k, v = rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    o, lse = oracle.attn_fwd(q, k, v, False)
    perm = RNG.permutation(N)
    o2, lse2 = oracle.attn_fwd(q, k[:, :, perm], v[:, :, perm], False)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    o3, lse3 = oracle.attn_fwd(q[:, :, perm], k, v, False)
    assert np.array_equal(o3, o[:, :, perm])
    assert np.array_equal(lse3, lse[:, :, perm])


def test_linear_in_v_and_weights_convex():
    """O is linear in V; with V = 1 every output is exactly a convex combination (= 1)."""
    B, H, N, D = 1, 2, 9, 8
    q, k = rand(B, H, N, D), rand(B, H, N, D)
    v1, v2 = rand(B, H, N, D), rand(B, H, N, D)
    for causal in (True, False):
        o1, l1 = oracle.attn_fwd(q, k, v1, causal)
        o2, _ = oracle.attn_fwd(q, k, v2, causal)
        o12, l12 = oracle.attn_fwd(q, k, v1 + 2.0 * v2, causal)
        np.testing.assert_allclose(o12, o1 + 2.0 * o2, atol=1e-12)
        assert np.array_equal(l12, l1)          # LSE does not depend on V
        ones, _ = oracle.attn_fwd(q, k, np.ones((B, H, N, D)), causal)
        np.testing.assert_allclose(ones, 1.0, atol=1e-14)


def test_heads_and_batches_are_independent():
    """Each (b, h) slice is computed from its own Q, K, V only."""
    B, H, N, D = 2, 3, 7, 8
    q, k, v = rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    o, lse = oracle.attn_fwd(q, k, v, True)
    for b in range(B):
        for h in range(H):
            o1, l1 = oracle.attn_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                     v[b:b + 1, h:h + 1], True)
            assert np.array_equal(o1[0, 0], o[b, h])
            assert np.array_equal(l1[0, 0], lse[b, h])


@pytest.mark.parametrize("causal", [True, False])
def test_lse_normalises_the_scores(causal):
    """sum_j exp(s_ij - lse_i) = 1 over the stage-1 scores of row i."""
    N, D = 20, 32
    q, k, v = rand(1, 1, N, D, scale=3.0), rand(1, 1, N, D, scale=3.0), rand(1, 1, N, D)
    _, lse = oracle.attn_fwd(q, k, v, causal)
    for i in range(N):
        s = oracle.attn_scores(q[0, 0], k[0, 0], causal, i)
        assert math.fsum(np.exp(s - lse[0, 0, i])) == pytest.approx(1.0, abs=1e-13)


@pytest.mark.parametrize("N,D,causal", [(1, 64, True), (33, 64, True), (70, 128, True),
                                        (65, 64, False), (17, 128, False)])
def test_matches_torch_sdpa_float64(N, D, causal):
    """Independent library routine: torch's CPU scaled_dot_product_attention in float64.

    LSE is checked against torch.logsumexp of torch's own float64 logits.
    """
    B, H = 2, 3
    q, k, v = rand(B, H, N, D, scale=2.0), rand(B, H, N, D, scale=2.0), rand(B, H, N, D)
    o, lse = oracle.attn_fwd(q, k, v, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    logits = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) / math.sqrt(D)
    if causal:
        mask = torch.ones(N, N, dtype=torch.bool).triu(1)
        logits = logits.masked_fill(mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------ grouped K/V heads

def gqa_sdpa_check(q, k, v, causal):
    """Oracle GQA against torch's float64 SDPA with its own grouped-head mapping."""
    o, lse = oracle.attn_fwd_gqa(q, k, v, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           enable_gqa=True)
    return np.abs(o - ref.numpy()).max()


@pytest.mark.parametrize("H,Hkv", [(6, 1), (6, 2), (6, 3), (8, 4)])
@pytest.mark.parametrize("causal", [True, False])
def test_gqa_matches_torch_sdpa_enable_gqa(H, Hkv, causal):
    """Independent library routine: torch SDPA with enable_gqa (query head h uses
    K/V head h // (H / Hkv)), float64 on the CPU."""
    B, N, D = 2, 19, 16
    q = rand(B, H, N, D, scale=2.0)
    k, v = rand(B, Hkv, N, D, scale=2.0), rand(B, Hkv, N, D)
    assert gqa_sdpa_check(q, k, v, causal) <= 1e-12


def test_gqa_with_one_group_per_head_is_attn_fwd():
    """Hkv = H reduces to plain attention, bit for bit."""
    q, k, v = rand(1, 4, 11, 8), rand(1, 4, 11, 8), rand(1, 4, 11, 8)
    o1, l1 = oracle.attn_fwd_gqa(q, k, v, True)
    o2, l2 = oracle.attn_fwd(q, k, v, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_gqa_head_map_and_rows_entry():
    """The head map of the KV-cache page (h_kv = floor(h / g)) on a worked case,
    and the row-subset entry point agreeing with the full one."""
    assert [oracle.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head(h, 6, 3) for h in range(6)] == [0, 0, 1, 1, 2, 2]
    assert [oracle.kv_head(h, 5, 1) for h in range(5)] == [0] * 5
    with pytest.raises(ValueError):
        oracle.kv_head(0, 6, 4)
    B, H, Hkv, N, D = 2, 4, 2, 9, 8
    q, k, v = rand(B, H, N, D), rand(B, Hkv, N, D), rand(B, Hkv, N, D)
    o, lse = oracle.attn_fwd_gqa(q, k, v, False)
    rows = [0, 8, 9, 40, 71]
    orow, lrow = oracle.attn_rows_gqa(q, k, v, False, rows)
    assert np.array_equal(orow, o.reshape(-1, D)[rows])
    assert np.array_equal(lrow, lse.reshape(-1)[rows])


def test_rows_entry_and_thread_count_are_bitwise_stable():
    """The row-subset entry point and any thread count give bit-identical results."""
    B, H, N, D = 1, 3, 40, 16
    q, k, v = rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    o1, l1 = oracle.attn_fwd(q, k, v, True, nthreads=1)
    o8, l8 = oracle.attn_fwd(q, k, v, True, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(l1, l8)
    rows = [0, 5, 39, 40, 79, 119]
    orow, lrow = oracle.attn_rows(q, k, v, True, rows, nthreads=3)
    flat_o, flat_l = o1.reshape(-1, D), l1.reshape(-1)
    assert np.array_equal(orow, flat_o[rows]) and np.array_equal(lrow, flat_l[rows])


def test_half_and_bfloat16_inputs_widen_exactly():
    """fp16 / bf16 tensors are widened to float64 without rounding."""
    x = torch.tensor([1.0, -2.5, 65504.0, 2.0 ** -24, 0.1], dtype=torch.float16)
    assert oracle.to_f64(x).tolist() == [float(t) for t in x.tolist()]
    y = torch.tensor([1.0, -3.0, 2.0 ** 100, 0.1, 3.0e38], dtype=torch.bfloat16)
    assert oracle.to_f64(y).tolist() == [float(t) for t in y.float().tolist()]


# ------------------------------------------------------------- row softmax

def test_softmax_rows_sum_to_one_and_shift_invariant():
    """Softmax study section 3.3: constant added to a row; rows sum to 1."""
    x = rand(37, 50, scale=4.0)
    y = oracle.row_softmax(x)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, atol=1e-14)
    shift = rand(37, 1, scale=100.0)
    np.testing.assert_allclose(oracle.row_softmax(x + shift), y, rtol=1e-12, atol=1e-15)


def test_softmax_all_zero_is_uniform():
    """Softmax study section 3.3: all-zero input gives 1/N everywhere."""
    for n in (1, 2, 257, 1000):
        y = oracle.row_softmax(np.zeros((3, n)))
        np.testing.assert_allclose(y, 1.0 / n, rtol=1e-15, atol=0)


def test_softmax_special_last_element_closed_form():
    """Last element 80 (softmax study section 3.3): y_last = 1/(1 + sum_{j<last} e^(x_j - 80))."""
    x = rand(5, 257)
    x[:, -1] = 80.0
    y = oracle.row_softmax(x)
    for r in range(5):
        rest = math.fsum(math.exp(t - 80.0) for t in x[r, :-1])
        assert y[r, -1] == pytest.approx(1.0 / (1.0 + rest), rel=1e-15)
        np.testing.assert_allclose(y[r, :-1], np.exp(x[r, :-1] - 80.0) * y[r, -1], rtol=1e-13)
    assert (y > 0).all()


def test_softmax_two_elements_logistic():
    a = np.array([-50.0, -1.0, 0.0, 3.0, 60.0])
    x = np.stack([a, np.zeros_like(a)], axis=1)
    y = oracle.row_softmax(x)
    np.testing.assert_allclose(y[:, 0], 1.0 / (1.0 + np.exp(-a)), rtol=1e-14)


def test_softmax_matches_library_routines():
    """Independent routines: scipy.special.softmax and torch.softmax in float64."""
    scipy_special = pytest.importorskip("scipy.special")
    x = rand(64, 333, scale=6.0)
    y = oracle.row_softmax(x)
    np.testing.assert_allclose(y, scipy_special.softmax(x, axis=1), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(y, torch.softmax(torch.from_numpy(x), dim=1).numpy(),
                               rtol=1e-13, atol=1e-300)


def test_softmax_rows_entry_matches_full():
    x = rand(20, 31)
    y = oracle.row_softmax(x, nthreads=1)
    rows = [0, 7, 19, 7]
    assert np.array_equal(oracle.row_softmax_rows(x, rows, nthreads=2), y[rows])
    assert np.array_equal(oracle.row_softmax(x, nthreads=8), y)


def test_wide_logit_spread_needs_the_row_max():
    """Logits 800 apart: exp of the spread overflows unless the row MAX is subtracted.

    The weight of the small logit underflows to 0, so O is exactly v of the
    large one and lse is exactly the large logit.
    """
    D = 4
    q = np.zeros((1, 1, 2, D))
    k = np.zeros((1, 1, 2, D))
    q[0, 0, 1, 0] = 2.0          # s_1j = 2*k_j0/2 = k_j0
    k[0, 0, 0, 0] = -400.0
    k[0, 0, 1, 0] = 400.0
    v = rand(1, 1, 2, D)
    o, lse = oracle.attn_fwd(q, k, v, True)
    assert np.array_equal(o[0, 0, 1], v[0, 0, 1])
    assert lse[0, 0, 1] == 400.0
    y = oracle.row_softmax(np.array([[-400.0, 400.0], [400.0, -400.0]]))
    assert np.array_equal(y, np.array([[0.0, 1.0], [1.0, 0.0]]))
