"""FP64 CPU oracle for attention forward and row softmax.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The product library never imports,
links or calls anything here, and nothing here imports the product package.

The arithmetic lives in ``oracle.c`` (plain C, double precision, compiled with
gcc into ``liboracle.so``).  This module only turns fp16 / bf16 / fp32 input
bits into exact float64 arrays and calls the C entry points.

Definitions followed (see the header of ``oracle.c`` for the stage-by-stage
statement):

* attention: "CUDA FlashAttention: from online softmax to long-sequence IO
  limits" (chengzipai.xyz), section 1 (O = softmax(QK^T/sqrt(D) + M)V, causal
  mask j <= i) and section 3 (the naive three stages);
* row softmax: the softmax kernel study (lpnh.cn/news/2830604), section 3.1
  (double-precision stable softmax as the CPU reference);
* attention backward: the gradients of the attention definition (the FA
  page, section 7, only says the LSE is kept for the backward pass); with
  grouped K/V heads, the sum of those gradients over each group (the chain
  rule through the KV page's section 3 head mapping);
* paged decode: "CUDA KV Cache: paged storage and long-context decode"
  (chengzipai.xyz), sections 2 (page-table addressing), 3 (query-head groups
  share a K/V head) and 5 (attention of the new token over the cached ones).

Pins: every function here is checked in ``tests/test_oracle.py`` against
closed forms, invariants and independent library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_I64 = ctypes.c_int64
_PD = ctypes.POINTER(ctypes.c_double)
_PI64 = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (host code only; no GPU involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    lib.oracle_attn_fwd.argtypes = [_PD, _PD, _PD, _PD, _PD, _I64, _I64, _I64, _I64,
                                    ctypes.c_int, ctypes.c_int]
    lib.oracle_attn_fwd.restype = ctypes.c_int
    lib.oracle_attn_bwd.argtypes = [_PD, _PD, _PD, _PD, _I64, _I64, _I64, _I64, ctypes.c_int,
                                    _PI64, _I64, _PD, _PD, _PD, ctypes.c_int]
    lib.oracle_attn_bwd.restype = ctypes.c_int
    lib.oracle_paged_decode.argtypes = [_PD, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                        _PI64, _I64, _PD, _PD, ctypes.c_int]
    lib.oracle_paged_decode.restype = ctypes.c_int
    lib.oracle_bits_to_double.argtypes = [ctypes.c_void_p, ctypes.c_int, _I64, _PD]
    lib.oracle_bits_to_double.restype = ctypes.c_int
    lib.oracle_attn_rows.argtypes = [_PD, _PD, _PD, _I64, _I64, _I64, _I64, ctypes.c_int,
                                     _PI64, _I64, _PD, _PD, ctypes.c_int]
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_attn_scores.argtypes = [_PD, _PD, _I64, _I64, ctypes.c_int, _I64, _PD]
    lib.oracle_attn_scores.restype = ctypes.c_int64
    lib.oracle_row_softmax.argtypes = [_PD, _PD, _I64, _I64, ctypes.c_int]
    lib.oracle_row_softmax.restype = ctypes.c_int
    lib.oracle_row_softmax_rows.argtypes = [_PD, _I64, _I64, _PI64, _I64, _PD,
                                            ctypes.c_int]
    lib.oracle_row_softmax_rows.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _bind(_LIB)
    return _lib


def swap_library(path: str | None):
    """Point this module at another build of the oracle (None: the default one).

    Used by the tests that plant mistakes in a copy of oracle.c and check that
    the pins catch them.  Returns nothing; not thread-safe.
    """
    global _lib
    with _lock:
        _lib = None if path is None else _bind(path)


def default_threads() -> int:
    """Threads the oracle uses: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------- conversions

def to_f64(a) -> np.ndarray:
    """Exact float64 copy of a host array or CPU torch tensor.

    fp16 and fp32 convert through numpy; bf16 is widened by placing its 16
    bits in the high half of an fp32 word, which is exact.
    """
    if hasattr(a, "detach"):  # torch tensor (CPU)
        import torch
        t = a.detach().contiguous()
        if t.dtype == torch.bfloat16:
            bits = t.view(torch.int16).numpy().astype(np.uint16)
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        a = t.numpy()
    a = np.asarray(a)
    if a.dtype == np.float64:
        return np.ascontiguousarray(a)
    return np.ascontiguousarray(a.astype(np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_PD)


# ----------------------------------------------------------------- attention

def attn_fwd(q, k, v, causal: bool, nthreads: int | None = None):
    """O [B,H,N,D] and LSE [B,H,N] in float64 for inputs [B,H,N,D]."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H, N, D = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    o = np.empty((B, H, N, D), np.float64)
    lse = np.empty((B, H, N), np.float64)
    rc = _load().oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, D,
                                 int(bool(causal)), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_attn_fwd failed (%d)" % rc)
    return o, lse


def attn_rows(q, k, v, causal: bool, rows, nthreads: int | None = None):
    """O and LSE for selected rows only; rows are flat ids (b*H+h)*N+i.

    Returns o [len(rows), D] and lse [len(rows)] in float64.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H, N, D = q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    o = np.empty((rows.size, D), np.float64)
    lse = np.empty((rows.size,), np.float64)
    rc = _load().oracle_attn_rows(_ptr(q), _ptr(k), _ptr(v), B, H, N, D, int(bool(causal)),
                                  rows.ctypes.data_as(_PI64), rows.size, _ptr(o), _ptr(lse),
                                  nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_attn_rows failed (%d)" % rc)
    return o, lse


def attn_bwd(q, k, v, dout, causal: bool, heads=None, nthreads: int | None = None):
    """Gradients dQ, dK, dV of sum(O * dout) for O = attention(q, k, v).

    Inputs [B,H,N,D] (any float type).  heads: flat head ids b*H + h to
    compute (all if None).  Returns three float64 arrays [len(heads), N, D]
    (reshaped to [B,H,N,D] when heads is None).
    """
    q, k, v, dout = to_f64(q), to_f64(k), to_f64(v), to_f64(dout)
    B, H, N, D = q.shape
    for x in (k, v, dout):
        assert x.shape == q.shape
    all_heads = heads is None
    heads = np.arange(B * H) if all_heads else heads
    heads = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
    dq = np.empty((heads.size, N, D), np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    rc = _load().oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, N, D,
                                 int(bool(causal)), heads.ctypes.data_as(_PI64), heads.size,
                                 _ptr(dq), _ptr(dk), _ptr(dv), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_attn_bwd failed (%d)" % rc)
    if all_heads:
        return dq.reshape(B, H, N, D), dk.reshape(B, H, N, D), dv.reshape(B, H, N, D)
    return dq, dk, dv


def kv_head(h: int, H: int, Hkv: int) -> int:
    """K/V head read by query head h when H query heads share Hkv K/V heads.

    "CUDA KV Cache: paged storage and long-context decode" (chengzipai.xyz),
    section 3: with g = H / Hkv query heads per group, query head h reads K/V
    head floor(h / g).
    """
    if Hkv < 1 or H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    return h // (H // Hkv)


def _kv_for_query_heads(x, H: int) -> np.ndarray:
    """[B, Hkv, N, D] -> [B, H, N, D]: slot h holds K/V head kv_head(h)."""
    x = to_f64(x)
    Hkv = x.shape[1]
    return np.ascontiguousarray(x[:, [kv_head(h, H, Hkv) for h in range(H)]])


def attn_fwd_gqa(q, k, v, causal: bool, nthreads: int | None = None):
    """Grouped-query attention: q [B,H,N,D], k and v [B,Hkv,N,D].

    Each query head is plain attention (attn_fwd) against its group's K/V head.
    """
    H = q.shape[1]
    return attn_fwd(q, _kv_for_query_heads(k, H), _kv_for_query_heads(v, H), causal, nthreads)


def attn_rows_gqa(q, k, v, causal: bool, rows, nthreads: int | None = None):
    """attn_rows for grouped K/V heads; rows are flat ids (b*H+h)*N+i of the query."""
    H = q.shape[1]
    return attn_rows(q, _kv_for_query_heads(k, H), _kv_for_query_heads(v, H), causal, rows,
                     nthreads)


def attn_bwd_gqa(q, k, v, dout, causal: bool, kv_heads=None, nthreads: int | None = None):
    """Gradients of sum(O * dout) for grouped-query attention (attn_fwd_gqa).

    q, dout [B,H,N,D]; k, v [B,Hkv,N,D].  Query head h of batch b reads K/V
    head kv_head(h) (KV page, section 3), so by the chain rule dQ_h is the
    plain backward of head h against that K/V head, and dK, dV of a K/V head
    are the sums over its group of the per-query-head dK, dV.

    kv_heads: flat K/V head ids b*Hkv + j to compute (all if None).  Returns
    (dq, dk, dv): dq [B,H,N,D] and dk, dv [B,Hkv,N,D] when kv_heads is None;
    otherwise dq [len(kv_heads)*g, N, D] (the group's query heads in order)
    and dk, dv [len(kv_heads), N, D].
    """
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    g = H // Hkv
    if Hkv < 1 or H % Hkv or k.shape != (B, Hkv, N, D) or v.shape != k.shape:
        raise ValueError("k, v must be [B, Hkv, N, D] with Hkv dividing H")
    all_kv = kv_heads is None
    kv_heads = np.arange(B * Hkv) if all_kv else np.asarray(kv_heads, dtype=np.int64)
    heads = np.asarray([(f // Hkv) * H + (f % Hkv) * g + i for f in kv_heads for i in range(g)],
                       dtype=np.int64)
    dq, dk_h, dv_h = attn_bwd(q, _kv_for_query_heads(k, H), _kv_for_query_heads(v, H), dout,
                              causal, heads=heads, nthreads=nthreads)
    dk = dk_h.reshape(len(kv_heads), g, N, D).sum(axis=1)
    dv = dv_h.reshape(len(kv_heads), g, N, D).sum(axis=1)
    if all_kv:
        return dq.reshape(B, H, N, D), dk.reshape(B, Hkv, N, D), dv.reshape(B, Hkv, N, D)
    return dq, dk, dv


def attn_scores(q, k, causal: bool, i: int) -> np.ndarray:
    """Stage 1 alone: the scaled scores of query row i of one head ([N,D] inputs)."""
    q, k = to_f64(q), to_f64(k)
    N, D = q.shape
    s = np.empty((N,), np.float64)
    n = _load().oracle_attn_scores(_ptr(q), _ptr(k), N, D, int(bool(causal)), int(i), _ptr(s))
    if n < 0:
        raise RuntimeError("oracle_attn_scores failed")
    return s[:n].copy()


# -------------------------------------------------------------- paged decode

def _bits16(a):
    """(uint16 bits, is_bf16) of a CPU torch fp16/bf16 tensor or a numpy float16 array."""
    if hasattr(a, "detach"):
        import torch
        t = a.detach().contiguous()
        if t.dtype not in (torch.float16, torch.bfloat16):
            raise TypeError("the cache must be fp16 or bf16")
        return np.ascontiguousarray(t.view(torch.int16).numpy().view(np.uint16)), \
            int(t.dtype == torch.bfloat16)
    a = np.ascontiguousarray(np.asarray(a))
    if a.dtype != np.float16:
        raise TypeError("the cache must be fp16 or bf16")
    return a.view(np.uint16), 0


def bits_to_f64(a) -> np.ndarray:
    """The cache converter used by paged_decode (exact decoding in oracle.c)."""
    bits, is_bf16 = _bits16(a)
    out = np.empty(bits.shape, np.float64)
    if _load().oracle_bits_to_double(bits.ctypes.data, is_bf16, bits.size, _ptr(out)) != 0:
        raise RuntimeError("oracle_bits_to_double failed")
    return out


def paged_decode(q, cache, block_table, lengths, page_size: int, rows=None,
                 nthreads: int | None = None):
    """Paged grouped-query decode in float64.

    q [B, Hq, D] (any float type), cache [P, 2, T, Hkv, D] fp16/bf16 (CPU),
    block_table [B, max_pages] and lengths [B] integers.  rows: flat ids
    b*Hq + h to compute (all if None).  Returns o [len(rows), D] and
    lse [len(rows)]; invalid requests get NaN.
    """
    qd = to_f64(q)
    B, Hq, D = qd.shape
    bits, is_bf16 = _bits16(cache)
    P, two, T, Hkv, Dc = bits.shape
    if two != 2 or T != page_size or Dc != D:
        raise ValueError("cache must be [P, 2, page_size, Hkv, D]")
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    if bt.ndim != 2 or bt.shape[0] != B or ln.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and lengths [B]")
    if rows is None:
        rows = np.arange(B * Hq)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    o = np.empty((rows.size, D), np.float64)
    lse = np.empty((rows.size,), np.float64)
    rc = _load().oracle_paged_decode(_ptr(qd), bits.ctypes.data, is_bf16, bt.ctypes.data,
                                     ln.ctypes.data, B, Hq, Hkv, D, T, P, bt.shape[1],
                                     rows.ctypes.data_as(_PI64), rows.size, _ptr(o), _ptr(lse),
                                     nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_paged_decode failed (%d)" % rc)
    return o, lse


# --------------------------------------------------------------- row softmax

def row_softmax(x, nthreads: int | None = None) -> np.ndarray:
    """y = softmax over the last axis of a 2-D x, in float64."""
    x = to_f64(x)
    M, N = x.shape
    y = np.empty((M, N), np.float64)
    rc = _load().oracle_row_softmax(_ptr(x), _ptr(y), M, N, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_row_softmax failed (%d)" % rc)
    return y


def row_softmax_rows(x, rows, nthreads: int | None = None) -> np.ndarray:
    """Softmax of the selected rows of x; returns [len(rows), N] float64."""
    x = to_f64(x)
    M, N = x.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    y = np.empty((rows.size, N), np.float64)
    rc = _load().oracle_row_softmax_rows(_ptr(x), M, N, rows.ctypes.data_as(_PI64), rows.size,
                                         _ptr(y), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_row_softmax_rows failed (%d)" % rc)
    return y
