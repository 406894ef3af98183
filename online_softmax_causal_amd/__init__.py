"""Python binding of libosc_attn.so: attention forward and row softmax on MI355X.

Argument marshalling only.  Every step of both operations runs in the HIP
kernels of the shared library; there is no Python, PyTorch or CPU fallback.
If the library has not been built (``python -m online_softmax_causal_amd.build``)
``load()`` raises.

The entry points mirror the C ABI in ``include/osc_attn.h``:

    attn_fwd(q, k, v, o, lse, B, H, N, D, causal, dtype, stream=None)
    row_softmax(x, y, M, N, stream=None)
    attn_fwd_gqa(q, k, v, o, lse, B, H, Hkv, N, D, causal, dtype, stream=None)
    attn_fwd_splitkv(q, k, v, o, lse, B, H, Hkv, N, D, causal, dtype, num_splits,
                     workspace, workspace_bytes, stream=None)
    attn_fwd_splitkv_workspace(B, H, N, D, causal, num_splits=0)
    paged_decode(q, cache, block_table, lengths, o, lse, B, Hq, Hkv, D, page_size,
                 num_pages, max_pages, dtype, num_splits, workspace, workspace_bytes,
                 stream=None)
    paged_decode_workspace(B, Hq, Hkv, D, page_size, max_pages, num_splits=0)
    paged_decode_noalloc(q, cache, block_table, lengths, o, lse, B, Hq, Hkv, D, page_size,
                         num_pages, max_pages, dtype, num_splits, stream=None)
    attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, causal, dtype, workspace,
             workspace_bytes, stream=None)
    attn_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, D, causal, dtype,
                 workspace, workspace_bytes, stream=None)
    attn_bwd_workspace(B, H, N)
    attn_status_str(status)

Pointer arguments accept device tensors or plain integer addresses.  A tensor
argument is checked before anything is enqueued: it must live on the same GPU
as the first tensor of the call, be contiguous, have the dtype the entry point
expects (q, k, v, dout and the cache in the 16-bit `dtype`; o, lse and the
gradients FP32; block_table and lengths int32) and hold at least as many
elements as the sizes imply; otherwise ValueError is raised.  (A CPU tensor
would hand the kernel a host address, and a short buffer would be written past
its end.)  An integer address is passed through unchecked.  The C call runs
with the tensors' device made current.  ``stream`` accepts None (PyTorch's
current stream on that device), a ``torch.cuda.Stream`` or an integer handle.  A nonzero
status raises ``AttnError``.  ``attention(q, k, v, causal)`` is a convenience
wrapper that allocates O and LSE with PyTorch and calls ``attn_fwd``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libosc_attn.so")

ATTN_F16 = 0
ATTN_BF16 = 1
PAGED_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # include/osc_attn.h
STATUS = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL",
    2: "ATTN_ERR_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_ALIGN",
    5: "ATTN_ERR_LAUNCH",
    6: "ATTN_ERR_ALIAS",
    7: "ATTN_ERR_WORKSPACE",
}
EXPORTS = ("attn_fwd", "attn_fwd_gqa", "attn_fwd_splitkv", "attn_fwd_splitkv_workspace",
           "paged_decode", "paged_decode_workspace", "paged_decode_noalloc", "attn_bwd",
           "attn_bwd_gqa", "attn_bwd_workspace", "row_softmax", "attn_status_str")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, STATUS.get(status, status),
                                          attn_status_str(status)))


def load():
    """Load libosc_attn.so and declare its signatures (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libosc_attn.so is not built: run "
                           "`python -m online_softmax_causal_amd.build` first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int,
                                 ctypes.c_int, vp]
    lib.attn_fwd_gqa.restype = ctypes.c_int
    lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, vp, i64, vp]
    lib.attn_fwd_splitkv.restype = ctypes.c_int
    lib.attn_fwd_splitkv_workspace.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.attn_fwd_splitkv_workspace.restype = i64
    lib.paged_decode.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                 ctypes.c_int, ctypes.c_int, vp, i64, vp]
    lib.paged_decode.restype = ctypes.c_int
    lib.paged_decode_workspace.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int]
    lib.paged_decode_workspace.restype = i64
    lib.paged_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                         i64, ctypes.c_int, ctypes.c_int, vp]
    lib.paged_decode_noalloc.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                             ctypes.c_int, vp, i64, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                 ctypes.c_int, ctypes.c_int, vp, i64, vp]
    lib.attn_bwd_gqa.restype = ctypes.c_int
    lib.attn_bwd_workspace.argtypes = [i64, i64, i64]
    lib.attn_bwd_workspace.restype = i64
    lib.row_softmax.argtypes = [vp, vp, i64, i64, vp]
    lib.row_softmax.restype = ctypes.c_int
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError("expected a tensor, an int address or None, got %r" % type(x))


def _check(where, args):
    """Validate the tensor arguments of one call before any launch; returns
    their common device (None if every argument is an address or None).

    args: (name, value, kind, numel) with kind "h" (the 16-bit dtype of the
    call), "f32" or "i32"; numel the element count the sizes imply.  Integer
    addresses and None are left to the C layer.
    """
    import torch
    want = {"f32": torch.float32, "i32": torch.int32}
    dev = None
    for name, t, kind, numel in args:
        if t is None or isinstance(t, int):
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s: %s must be a tensor, an int address or None" % (where, name))
        if kind == "h":
            if t.dtype not in (torch.float16, torch.bfloat16):
                raise ValueError("%s: %s must be float16 or bfloat16, got %s" % (where, name, t.dtype))
        elif kind != "bytes" and t.dtype != want[kind]:
            raise ValueError("%s: %s must be %s, got %s" % (where, name, want[kind], t.dtype))
        if kind == "bytes":
            have = t.numel() * t.element_size()
            if have < numel:
                raise ValueError("%s: %s holds %d bytes, the call needs %d" % (where, name, have, numel))
        elif t.numel() < numel:
            raise ValueError("%s: %s holds %d elements, the sizes need %d" % (where, name, t.numel(), numel))
        if not t.is_contiguous():
            raise ValueError("%s: %s must be contiguous" % (where, name))
    for name, t, _, _ in args:
        if t is None or isinstance(t, int):
            continue
        if not t.is_cuda:
            raise ValueError("%s: %s is on %s, not on a GPU" % (where, name, t.device))
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s: %s is on %s, other arguments on %s" % (where, name, t.device, dev))
    return dev


def _check_half_dtype(where, dtype, tensors):
    """The 16-bit tensors of a call must match its dtype argument."""
    import torch
    code = _dtype(dtype)
    td = {ATTN_F16: torch.float16, ATTN_BF16: torch.bfloat16}.get(code)
    for name, t in tensors:
        if isinstance(t, torch.Tensor) and td is not None and t.dtype != td:
            raise ValueError("%s: %s is %s but dtype says %s" % (where, name, t.dtype, td))


def _on(dev):
    """The context a call runs in: the device of its tensors made current (the
    library launches on the current device and keeps its per-device state
    there); no change when every argument is a raw address."""
    if dev is None:
        return contextlib.nullcontext()
    import torch
    return torch.cuda.device(dev)


def _stream(s, dev=None):
    if s is None:
        import torch
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    raise TypeError("expected a stream handle, torch.cuda.Stream or None")


def _dtype(d) -> int:
    if isinstance(d, int):
        return d
    if isinstance(d, str):
        return {"f16": ATTN_F16, "fp16": ATTN_F16, "float16": ATTN_F16,
                "bf16": ATTN_BF16, "bfloat16": ATTN_BF16}[d]
    import torch
    return {torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}[d]


def attn_status_str(status: int) -> str:
    return load().attn_status_str(int(status)).decode()


def attn_fwd(q, k, v, o, lse, B, H, N, D, causal, dtype, stream=None) -> None:
    """Enqueue attention forward (see include/osc_attn.h); raises AttnError on a bad status."""
    n = int(B) * int(H) * int(N)
    _check_half_dtype("attn_fwd", dtype, [("q", q), ("k", k), ("v", v)])
    dev = _check("attn_fwd", [("q", q, "h", n * int(D)), ("k", k, "h", n * int(D)), ("v", v, "h", n * int(D)),
                              ("o", o, "f32", n * int(D)), ("lse", lse, "f32", n)])
    with _on(dev):
        st = load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(N),
                             int(D), int(bool(causal)), _dtype(dtype), _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_fwd")


def attn_fwd_gqa(q, k, v, o, lse, B, H, Hkv, N, D, causal, dtype, stream=None) -> None:
    """Enqueue grouped-query attention forward (K/V have Hkv heads, Hkv divides H)."""
    n, nk = int(B) * int(H) * int(N), int(B) * int(Hkv) * int(N)
    _check_half_dtype("attn_fwd_gqa", dtype, [("q", q), ("k", k), ("v", v)])
    dev = _check("attn_fwd_gqa", [("q", q, "h", n * int(D)), ("k", k, "h", nk * int(D)),
                                  ("v", v, "h", nk * int(D)), ("o", o, "f32", n * int(D)),
                                  ("lse", lse, "f32", n)])
    with _on(dev):
        st = load().attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                 int(Hkv), int(N), int(D), int(bool(causal)), _dtype(dtype),
                                 _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_fwd_gqa")


def attn_fwd_splitkv_workspace(B, H, N, D, causal, num_splits=0) -> int:
    """Workspace bytes attn_fwd_splitkv needs (0: one segment, no workspace); -1 if invalid."""
    return int(load().attn_fwd_splitkv_workspace(int(B), int(H), int(N), int(D),
                                                 int(bool(causal)), int(num_splits)))


def attn_fwd_splitkv(q, k, v, o, lse, B, H, Hkv, N, D, causal, dtype, num_splits, workspace,
                     workspace_bytes, stream=None) -> None:
    """Enqueue split-KV attention forward (partial states in `workspace`, then a merge)."""
    n, nk = int(B) * int(H) * int(N), int(B) * int(Hkv) * int(N)
    _check_half_dtype("attn_fwd_splitkv", dtype, [("q", q), ("k", k), ("v", v)])
    dev = _check("attn_fwd_splitkv", [("q", q, "h", n * int(D)), ("k", k, "h", nk * int(D)),
                                      ("v", v, "h", nk * int(D)), ("o", o, "f32", n * int(D)),
                                      ("lse", lse, "f32", n),
                                      ("workspace", workspace, "bytes", max(0, int(workspace_bytes)))])
    with _on(dev):
        st = load().attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                     int(Hkv), int(N), int(D), int(bool(causal)), _dtype(dtype),
                                     int(num_splits), _ptr(workspace), int(workspace_bytes),
                                     _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_fwd_splitkv")


def paged_decode_workspace(B, Hq, Hkv, D, page_size, max_pages, num_splits=0) -> int:
    """Workspace bytes paged_decode needs (0: one segment, no workspace); -1 if invalid."""
    return int(load().paged_decode_workspace(int(B), int(Hq), int(Hkv), int(D), int(page_size),
                                             int(max_pages), int(num_splits)))


def paged_decode(q, cache, block_table, lengths, o, lse, B, Hq, Hkv, D, page_size, num_pages,
                 max_pages, dtype, num_splits, workspace, workspace_bytes, stream=None) -> None:
    """Enqueue one paged grouped-query decode step (block_table, lengths: int32 device)."""
    nq = int(B) * int(Hq)
    _check_half_dtype("paged_decode", dtype, [("q", q), ("cache", cache)])
    dev = _check("paged_decode", [("q", q, "h", nq * int(D)),
                                  ("cache", cache, "h",
                                   int(num_pages) * 2 * int(page_size) * int(Hkv) * int(D)),
                                  ("block_table", block_table, "i32", int(B) * int(max_pages)),
                                  ("lengths", lengths, "i32", int(B)), ("o", o, "f32", nq * int(D)),
                                  ("lse", lse, "f32", nq),
                                  ("workspace", workspace, "bytes", max(0, int(workspace_bytes)))])
    with _on(dev):
        st = load().paged_decode(_ptr(q), _ptr(cache), _ptr(block_table), _ptr(lengths), _ptr(o),
                                 _ptr(lse), int(B), int(Hq), int(Hkv), int(D), int(page_size),
                                 int(num_pages), int(max_pages), _dtype(dtype), int(num_splits),
                                 _ptr(workspace), int(workspace_bytes), _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "paged_decode")


def paged_decode_noalloc(q, cache, block_table, lengths, o, lse, B, Hq, Hkv, D, page_size,
                         num_pages, max_pages, dtype, num_splits, stream=None) -> None:
    """paged_decode without a workspace: the segment states go to the library's
    fixed per-device array of PAGED_NOALLOC_SCRATCH_BYTES bytes."""
    nq = int(B) * int(Hq)
    _check_half_dtype("paged_decode_noalloc", dtype, [("q", q), ("cache", cache)])
    dev = _check("paged_decode_noalloc", [
        ("q", q, "h", nq * int(D)),
        ("cache", cache, "h", int(num_pages) * 2 * int(page_size) * int(Hkv) * int(D)),
        ("block_table", block_table, "i32", int(B) * int(max_pages)),
        ("lengths", lengths, "i32", int(B)), ("o", o, "f32", nq * int(D)), ("lse", lse, "f32", nq)])
    with _on(dev):
        st = load().paged_decode_noalloc(_ptr(q), _ptr(cache), _ptr(block_table), _ptr(lengths),
                                         _ptr(o), _ptr(lse), int(B), int(Hq), int(Hkv), int(D),
                                         int(page_size), int(num_pages), int(max_pages), _dtype(dtype),
                                         int(num_splits), _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "paged_decode_noalloc")


def _check_bwd(where, q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, D, dtype, workspace,
               workspace_bytes):
    n, nk = int(B) * int(H) * int(N), int(B) * int(Hkv) * int(N)
    d = int(D)
    _check_half_dtype(where, dtype, [("q", q), ("k", k), ("v", v), ("dout", dout)])
    return _check(where, [("q", q, "h", n * d), ("k", k, "h", nk * d), ("v", v, "h", nk * d),
                          ("o", o, "f32", n * d), ("lse", lse, "f32", n), ("dout", dout, "h", n * d),
                          ("dq", dq, "f32", n * d), ("dk", dk, "f32", nk * d), ("dv", dv, "f32", nk * d),
                          ("workspace", workspace, "bytes", max(0, int(workspace_bytes)))])


def attn_bwd_workspace(B, H, N) -> int:
    """Workspace bytes attn_bwd needs (8 * B*H*N); -1 if invalid."""
    return int(load().attn_bwd_workspace(int(B), int(H), int(N)))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, causal, dtype, workspace,
             workspace_bytes, stream=None) -> None:
    """Enqueue attention backward (dq, dk, dv FP32) from the forward's o and lse."""
    dev = _check_bwd("attn_bwd", q, k, v, o, lse, dout, dq, dk, dv, B, H, H, N, D, dtype,
                     workspace, workspace_bytes)
    with _on(dev):
        st = load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                             _ptr(dk), _ptr(dv), int(B), int(H), int(N), int(D), int(bool(causal)),
                             _dtype(dtype), _ptr(workspace), int(workspace_bytes), _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_bwd")


def attn_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, D, causal, dtype, workspace,
                 workspace_bytes, stream=None) -> None:
    """Enqueue attention backward with Hkv shared K/V heads (k, v, dk, dv [B, Hkv, N, D])."""
    dev = _check_bwd("attn_bwd_gqa", q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, D, dtype,
                     workspace, workspace_bytes)
    with _on(dev):
        st = load().attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                 _ptr(dk), _ptr(dv), int(B), int(H), int(Hkv), int(N), int(D),
                                 int(bool(causal)), _dtype(dtype), _ptr(workspace),
                                 int(workspace_bytes), _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_bwd_gqa")


def row_softmax(x, y, M, N, stream=None) -> None:
    """Enqueue the row softmax of an FP32 [M, N] matrix; raises AttnError on a bad status."""
    dev = _check("row_softmax", [("x", x, "f32", int(M) * int(N)), ("y", y, "f32", int(M) * int(N))])
    with _on(dev):
        st = load().row_softmax(_ptr(x), _ptr(y), int(M), int(N), _stream(stream, dev))
    if st != 0:
        raise AttnError(st, "row_softmax")


def attention(q, k, v, causal: bool, stream=None):
    """O (FP32) and LSE (FP32) for contiguous device tensors q, k, v of shape [B, H, N, D]."""
    import torch
    B, H, N, D = q.shape
    if not q.is_cuda:
        raise ValueError("attention: q is on %s, not on a GPU" % q.device)
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, N, D]")
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    o = torch.empty((B, H, N, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, o, lse, B, H, N, D, causal, q.dtype, stream)
    return o, lse
