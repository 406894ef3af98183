"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module draws random inputs and describes workload shapes.  It holds none
of the method's arithmetic: no scores, no softmax, no reductions.  Both the
HIP path's callers and the oracle's callers take their inputs from here.

Recipe (the same for every workload): a torch CPU ``Generator`` seeded with
the workload's seed draws float32 ``randn`` for Q, then K, then V (in that
order), each scaled by its standard deviation, then rounded to the storage
dtype with torch's round-to-nearest-even cast.  Row-softmax inputs are float32
``randn`` with the last element of every row overwritten by a special value
(the softmax kernel study, lpnh.cn/news/2830604, section 3.3, tests rows
whose last element is special; 80.0 forces the running maximum to jump at the
very end of the row).

The attention shapes follow "CUDA FlashAttention: from online softmax to
long-sequence IO limits" (chengzipai.xyz), section 1: B=1, H=32, D=128 with N
from 512 to 8192, causal fp16.  The row-softmax boundary shape M=1025, N=257
is the softmax study's section 3.4 case.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int
    H: int
    N: int
    D: int
    causal: bool
    dtype: str          # "f16" or "bf16"
    sigma_qk: float
    sigma_v: float
    seed: int
    Hkv: int | None = None   # K/V heads (grouped-query attention); None = H

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv is None else self.Hkv

    @property
    def flops(self) -> float:
        """Algorithmic FLOP: 2BHN^2D causal, 4BHN^2D non-causal (section 1 of the FA page)."""
        return attn_flops(self.B, self.H, self.N, self.D, self.causal)

    def describe(self) -> str:
        heads = "H%d" % self.H if self.Hkv is None else "Hq%d Hkv%d" % (self.H, self.Hkv)
        return "%s attn fwd %s B%d %s N%d D%d" % (
            "causal" if self.causal else "non-causal", self.dtype, self.B, heads, self.N, self.D)


@dataclass(frozen=True)
class SoftmaxWorkload:
    name: str
    M: int
    N: int
    last: float
    seed: int

    @property
    def bytes(self) -> float:
        """Algorithmic bytes: read x once and write y once, fp32."""
        return 8.0 * self.M * self.N

    def describe(self) -> str:
        return "row_softmax fp32 M%d N%d" % (self.M, self.N)


def attn_flops(B: int, H: int, N: int, D: int, causal: bool) -> float:
    return (2.0 if causal else 4.0) * B * H * N * N * D


ATTN = {
    "C1": AttnWorkload("C1", 1, 4, 256, 128, True, "f16", 1.0, 1.0, 43),
    "C2": AttnWorkload("C2", 1, 32, 512, 128, True, "f16", 1.0, 1.0, 44),
    "C3": AttnWorkload("C3", 1, 32, 2048, 128, True, "bf16", 3.0, 1.0, 45),
    "C4": AttnWorkload("C4", 1, 32, 8192, 128, True, "f16", 1.0, 1.0, 46),
    "C5": AttnWorkload("C5", 4, 32, 4095, 64, False, "bf16", 1.0, 1.0, 47),
}

# The rest of the FA page's sequence-length sweep (section 8: B=1, H=32,
# D=128, causal, fp16, N = 512 ... 8192); N = 512 and 8192 are C2 and C4.
SWEEP = {
    "F1K": AttnWorkload("F1K", 1, 32, 1024, 128, True, "f16", 1.0, 1.0, 53),
    "F2K": AttnWorkload("F2K", 1, 32, 2048, 128, True, "f16", 1.0, 1.0, 54),
    "F4K": AttnWorkload("F4K", 1, 32, 4096, 128, True, "f16", 1.0, 1.0, 55),
}

# Grouped-query attention: 32 query heads sharing 8 K/V heads at D=128 (the
# head configuration of the KV-cache page's decode measurements, section 3),
# at the FA page's longest prefill length.
GQA = {
    "G1": AttnWorkload("G1", 1, 32, 8192, 128, True, "f16", 1.0, 1.0, 50, Hkv=8),
    "G2": AttnWorkload("G2", 2, 8, 1000, 64, False, "bf16", 2.0, 1.0, 51, Hkv=1),
}

# Long sequence, few heads: the case the FA page (section 7) splits along the
# keys for; without a split the grid covers one CU per query tile.
SPLITKV = {
    "S1": AttnWorkload("S1", 1, 2, 16384, 128, True, "f16", 1.0, 1.0, 52),
}

@dataclass(frozen=True)
class DecodeWorkload:
    """One paged grouped-query decode step ("CUDA KV Cache: paged storage and
    long-context decode" (chengzipai.xyz), section 8: B=8, Hq=32, Hkv=8,
    D=128, fp16, page size 16, context 1K to 32K, every request at the same
    context length)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    ctx: int
    dtype: str
    seed: int

    @property
    def max_pages(self) -> int:
        return (self.ctx + self.page_size - 1) // self.page_size

    @property
    def num_pages(self) -> int:
        """Cache pages: exactly the pages the requests use."""
        return self.B * self.max_pages

    @property
    def bytes(self) -> float:
        """Algorithmic bytes: K and V of every cached token read once, q read,
        o (FP32) and lse written."""
        kv = 2.0 * self.B * self.ctx * self.Hkv * self.D * 2
        return kv + self.B * self.Hq * self.D * (2 + 4) + self.B * self.Hq * 4

    def describe(self) -> str:
        return "paged GQA decode %s B%d Hq%d Hkv%d D%d page%d ctx%d" % (
            self.dtype, self.B, self.Hq, self.Hkv, self.D, self.page_size, self.ctx)


DECODE = {
    "D%d" % (ctx // 1024): DecodeWorkload("D%d" % (ctx // 1024), 8, 32, 8, 128, 16, ctx, "f16",
                                          60 + i)
    for i, ctx in enumerate((1024, 4096, 8192, 16384, 32768))
}

SOFTMAX = {
    "R1": SoftmaxWorkload("R1", 1025, 257, 80.0, 48),
    "R2": SoftmaxWorkload("R2", 8192, 32768, 80.0, 49),
}

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}


def attn_inputs(B: int, H: int, N: int, D: int, dtype: str, seed: int,
                sigma_qk: float = 1.0, sigma_v: float = 1.0):
    """Q, K, V as contiguous CPU tensors [B,H,N,D] of the storage dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (B, H, N, D)
    td = TORCH_DTYPE[dtype]
    q = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk).to(td)
    k = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk).to(td)
    v = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_v).to(td)
    return q.contiguous(), k.contiguous(), v.contiguous()


def gqa_inputs(B: int, H: int, Hkv: int, N: int, D: int, dtype: str, seed: int,
               sigma_qk: float = 1.0, sigma_v: float = 1.0):
    """Q [B,H,N,D] and K, V [B,Hkv,N,D] (same recipe and draw order as attn_inputs)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    td = TORCH_DTYPE[dtype]
    q = (torch.randn((B, H, N, D), generator=g, dtype=torch.float32) * sigma_qk).to(td)
    k = (torch.randn((B, Hkv, N, D), generator=g, dtype=torch.float32) * sigma_qk).to(td)
    v = (torch.randn((B, Hkv, N, D), generator=g, dtype=torch.float32) * sigma_v).to(td)
    return q.contiguous(), k.contiguous(), v.contiguous()


def bwd_inputs(B: int, H: int, N: int, D: int, dtype: str, seed: int, sigma_qk: float = 1.0,
               sigma_v: float = 1.0, sigma_do: float = 1.0):
    """Q, K, V as attn_inputs, then dO [B,H,N,D] ~ N(0, sigma_do^2) drawn after V."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (B, H, N, D)
    td = TORCH_DTYPE[dtype]
    q = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk).to(td)
    k = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk).to(td)
    v = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_v).to(td)
    do = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_do).to(td)
    return q.contiguous(), k.contiguous(), v.contiguous(), do.contiguous()


def bwd_gqa_inputs(B: int, H: int, Hkv: int, N: int, D: int, dtype: str, seed: int,
                   sigma_qk: float = 1.0, sigma_v: float = 1.0, sigma_do: float = 1.0):
    """q [B,H,N,D], k, v [B,Hkv,N,D], dO [B,H,N,D]; drawn in that order."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    td = TORCH_DTYPE[dtype]
    q = (torch.randn((B, H, N, D), generator=g, dtype=torch.float32) * sigma_qk).to(td)
    k = (torch.randn((B, Hkv, N, D), generator=g, dtype=torch.float32) * sigma_qk).to(td)
    v = (torch.randn((B, Hkv, N, D), generator=g, dtype=torch.float32) * sigma_v).to(td)
    do = (torch.randn((B, H, N, D), generator=g, dtype=torch.float32) * sigma_do).to(td)
    return q.contiguous(), k.contiguous(), v.contiguous(), do.contiguous()


def workload_inputs(w: AttnWorkload):
    if w.Hkv is not None:
        return gqa_inputs(w.B, w.H, w.Hkv, w.N, w.D, w.dtype, w.seed, w.sigma_qk, w.sigma_v)
    return attn_inputs(w.B, w.H, w.N, w.D, w.dtype, w.seed, w.sigma_qk, w.sigma_v)


def decode_inputs(B: int, Hq: int, Hkv: int, D: int, page_size: int, num_pages: int,
                  max_pages: int, lengths, dtype: str, seed: int, sigma_qk: float = 1.0,
                  sigma_v: float = 1.0):
    """q [B,Hq,D], cache [P,2,T,Hkv,D], block_table [B,max_pages] int32, lengths [B] int32.

    Draw order: q, then K pages, then V pages (each float32 randn times its
    sigma, rounded to the dtype); then one random permutation of the page
    ids, dealt to the requests row by row, so every request's pages are
    scattered over the cache (the page's Figure 1: logical pages map to
    arbitrary physical pages).  Table entries past num_pages repeat page ids.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    td = TORCH_DTYPE[dtype]
    q = (torch.randn((B, Hq, D), generator=g, dtype=torch.float32) * sigma_qk).to(td)
    shape = (num_pages, page_size, Hkv, D)
    k = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk).to(td)
    v = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_v).to(td)
    cache = torch.stack((k, v), dim=1).contiguous()
    del k, v
    perm = torch.randperm(num_pages, generator=g)
    flat = perm.repeat((B * max_pages + num_pages - 1) // num_pages)[:B * max_pages]
    block_table = flat.reshape(B, max_pages).to(torch.int32).contiguous()
    lengths = torch.as_tensor(list(lengths), dtype=torch.int32).contiguous()
    return q.contiguous(), cache, block_table, lengths


def decode_workload_inputs(w: DecodeWorkload):
    return decode_inputs(w.B, w.Hq, w.Hkv, w.D, w.page_size, w.num_pages, w.max_pages,
                         [w.ctx] * w.B, w.dtype, w.seed)


def softmax_inputs(M: int, N: int, seed: int, last: float | None = 80.0):
    """x [M,N] float32 CPU tensor; the last element of each row set to ``last``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn((M, N), generator=g, dtype=torch.float32)
    if last is not None:
        x[:, -1] = last
    return x.contiguous()


def sample_rows(B: int, H: int, N: int, count: int, seed: int):
    """Flat row ids (b*H+h)*N+i to check at full size.

    Always includes the first and last rows of the first and last heads and
    rows around multiples of 64 (tile edges), plus seeded random rows.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    BH = B * H
    count = min(count, BH * N)
    picks = set()
    for bh in {0, BH - 1}:
        for i in {0, 1, N // 2, N - 2, N - 1}:
            if 0 <= i < N:
                picks.add(bh * N + i)
    for e in range(64, N, max(64, (N // 8) // 64 * 64 or 64)):
        bh = int(torch.randint(0, BH, (1,), generator=g))
        for i in (e - 1, e):
            if 0 <= i < N:
                picks.add(bh * N + i)
    while len(picks) < count:
        picks.add(int(torch.randint(0, BH * N, (1,), generator=g)))
    return sorted(picks)
