"""Pins of the FP64 paged-decode oracle (CPU only).

The oracle follows "CUDA KV Cache: paged storage and long-context decode"
(chengzipai.xyz): section 2 (cache [P][2][T][Hkv][D]; logical token t of
request b is slot t mod T of page block_table[b][t / T]), section 3 (query
head h reads K/V head floor(h / g)) and section 5 (the new token's query
attends over every cached token).  Each test checks it against something
other than itself: the exact fp16/bf16 decodings of numpy and torch, the
attention oracle's last causal row on K/V gathered here with numpy indexing,
torch's float64 SDPA, closed forms and exact invariances.
"""
import numpy as np
import pytest
import torch

import oracle


def make_case(B=3, Hq=8, Hkv=2, D=64, T=4, P=40, lengths=(9, 1, 23), dtype=torch.float16,
              seed=0, sigma=1.0):
    """Random cache with every request's pages drawn without replacement."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g, dtype=torch.float32).to(dtype)
    cache = (torch.randn(P, 2, T, Hkv, D, generator=g, dtype=torch.float32) * sigma).to(dtype)
    max_pages = max((n + T - 1) // T for n in lengths) + 1
    perm = torch.randperm(P, generator=g).numpy()
    bt = np.full((B, max_pages), -1, np.int32)
    k = 0
    for b in range(B):
        for i in range(max_pages):
            bt[b, i] = perm[k % P]
            k += 1
    return q, cache, bt, np.asarray(lengths, np.int32), T


def gather(cache, bt, b, n, T, kind):
    """[Hkv, n, D] float64: the request's first n cached tokens, by numpy indexing."""
    c = oracle.to_f64(cache)
    t = np.arange(n)
    return np.ascontiguousarray(c[bt[b, t // T], kind, t % T].transpose(1, 0, 2))


# ----------------------------------------------------------- exact decoding

def test_fp16_bits_decode_exactly():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.bits_to_f64(bits.view(np.float16))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_bits_decode_exactly():
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    t = bits.view(torch.bfloat16)
    ref = t.to(torch.float64).numpy()
    got = oracle.bits_to_f64(t)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------- definitions

@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("T,Hkv", [(4, 2), (1, 1), (16, 4)])
def test_equals_last_causal_row_of_attention(dtype, T, Hkv):
    """Decode of request b = row len_b - 1 of causal attention over its tokens."""
    q, cache, bt, lens, T = make_case(T=T, Hkv=Hkv, Hq=4 * Hkv, dtype=dtype, P=48)
    B, Hq, D = q.shape
    o, lse = oracle.paged_decode(q, cache, bt, lens, T)
    for b in range(B):
        n = int(lens[b])
        kb = gather(cache, bt, b, n, T, 0)[None]
        vb = gather(cache, bt, b, n, T, 1)[None]
        qq = np.zeros((1, Hq, n, D))
        qq[0, :, n - 1] = oracle.to_f64(q)[b]
        rows = [h * n + n - 1 for h in range(Hq)]
        o_ref, lse_ref = oracle.attn_rows_gqa(qq, kb, vb, True, rows)
        np.testing.assert_allclose(o[b * Hq:(b + 1) * Hq], o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b * Hq:(b + 1) * Hq], lse_ref, rtol=0, atol=1e-12)


def test_matches_torch_sdpa_float64():
    q, cache, bt, lens, T = make_case(Hq=6, Hkv=3, D=64, T=8, P=30, lengths=(17, 40, 5))
    B, Hq, D = q.shape
    o, lse = oracle.paged_decode(q, cache, bt, lens, T)
    for b in range(B):
        n = int(lens[b])
        kb = torch.from_numpy(gather(cache, bt, b, n, T, 0))[None]
        vb = torch.from_numpy(gather(cache, bt, b, n, T, 1))[None]
        qb = torch.from_numpy(oracle.to_f64(q)[b])[None, :, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, enable_gqa=True)
        np.testing.assert_allclose(o[b * Hq:(b + 1) * Hq], ref[0, :, 0].numpy(), rtol=0,
                                   atol=1e-12)
        s = (qb @ torch.repeat_interleave(kb, Hq // kb.shape[1], dim=1).transpose(-1, -2)) / np.sqrt(D)
        np.testing.assert_allclose(lse[b * Hq:(b + 1) * Hq], torch.logsumexp(s, -1)[0, :, 0].numpy(),
                                   rtol=0, atol=1e-12)


def test_single_token_returns_v0_and_its_logit():
    q, cache, bt, lens, T = make_case(lengths=(1, 1, 1))
    B, Hq, D = q.shape
    g = Hq // cache.shape[3]
    o, lse = oracle.paged_decode(q, cache, bt, lens, T)
    c = oracle.to_f64(cache)
    qd = oracle.to_f64(q)
    for b in range(B):
        for h in range(Hq):
            k0 = c[bt[b, 0], 0, 0, h // g]
            v0 = c[bt[b, 0], 1, 0, h // g]
            assert np.array_equal(o[b * Hq + h], v0)
            assert abs(lse[b * Hq + h] - qd[b, h] @ k0 / np.sqrt(D)) < 1e-12


def test_identical_keys_give_the_mean_of_v():
    q, cache, bt, lens, T = make_case(lengths=(13, 7, 30))
    cache[:, 0] = cache[0, 0, 0]
    B, Hq, D = q.shape
    o, lse = oracle.paged_decode(q, cache, bt, lens, T)
    qd = oracle.to_f64(q)
    k = oracle.to_f64(cache)[0, 0, 0]
    g = Hq // cache.shape[3]
    for b in range(B):
        n = int(lens[b])
        v = gather(cache, bt, b, n, T, 1)
        for h in range(Hq):
            np.testing.assert_allclose(o[b * Hq + h], v[h // g].mean(0), rtol=0, atol=1e-12)
            s = qd[b, h] @ k[h // g] / np.sqrt(D)
            assert abs(lse[b * Hq + h] - (s + np.log(n))) < 1e-12


def test_physical_page_order_does_not_matter():
    """Moving pages in the cache and updating the table gives the same bits."""
    q, cache, bt, lens, T = make_case(P=40)
    o1, l1 = oracle.paged_decode(q, cache, bt, lens, T)
    perm = np.random.default_rng(3).permutation(cache.shape[0])
    moved = torch.empty_like(cache)
    moved[torch.from_numpy(perm)] = cache
    o2, l2 = oracle.paged_decode(q, moved, perm[bt].astype(np.int32), lens, T)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_heads_of_a_group_share_their_kv_head():
    q, cache, bt, lens, T = make_case(Hq=8, Hkv=2)
    q[:, 1] = q[:, 0]   # same group (g = 4)
    q[:, 4] = q[:, 0]   # next group
    o, _ = oracle.paged_decode(q, cache, bt, lens, T)
    o = o.reshape(3, 8, -1)
    assert np.array_equal(o[:, 0], o[:, 1])
    assert not np.allclose(o[:, 0], o[:, 4])


def test_invalid_requests_get_nan_and_others_are_unaffected():
    q, cache, bt, lens, T = make_case(B=5, lengths=(9, 0, 23, 6, 6), P=60)
    P = cache.shape[0]
    bt[2, 3] = P          # used by request 2 (tokens 12..15)
    bt[3, 4] = -7         # past request 3's last token: never read
    lens[4] = bt.shape[1] * T + 1
    o, lse = oracle.paged_decode(q, cache, bt, lens, T)
    Hq = q.shape[1]
    o = o.reshape(5, Hq, -1)
    lse = lse.reshape(5, Hq)
    for b in (1, 2, 4):
        assert np.isnan(o[b]).all() and np.isnan(lse[b]).all()
    for b in (0, 3):
        assert np.isfinite(o[b]).all() and np.isfinite(lse[b]).all()
    good = np.asarray([0, 3])
    o_ref, _ = oracle.paged_decode(q[good], cache, bt[good], lens[good], T)
    assert np.array_equal(o[good].reshape(-1, o.shape[-1]), o_ref)
