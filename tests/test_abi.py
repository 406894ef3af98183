"""The C ABI library on the CPU: it loads, exports what include/*.h declares,
and rejects bad arguments before any HIP call (no kernel is launched here)."""
import ctypes
import glob
import os
import re

import pytest

import online_softmax_causal_amd as osc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASE = 1 << 40          # a 256-byte aligned address that is never dereferenced
MB = 1 << 20


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(",
                         text, flags=re.M):
            if m.group(1) not in ("defined",):
                names.add(m.group(1))
    return names


def test_library_loads_and_exports_every_declared_symbol():
    lib = osc.load()
    names = declared_functions()
    assert {"attn_fwd", "row_softmax", "attn_status_str"} <= names
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_every_bound_entry_point_is_declared():
    """The binding calls nothing the header does not declare, and the header
    declares nothing the binding leaves out."""
    assert set(osc.EXPORTS) == declared_functions()


def test_ceiling_probe_library_loads_and_rejects_bad_arguments():
    """The matrix-core ceiling probe that bench.py --ceiling runs is a library
    of its own (not part of the declared interface): it loads, reports its
    sizes, and refuses bad arguments before anything is launched."""
    path = os.path.join(ROOT, "online_softmax_causal_amd", "libosc_ceiling.so")
    assert os.path.exists(path), "run python -m online_softmax_causal_amd.build"
    lib = ctypes.CDLL(path)
    lib.osc_ceiling_src_bytes.restype = ctypes.c_int64
    lib.osc_ceiling_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]
    assert lib.osc_ceiling_src_bytes() == 6144 * 16
    lib.osc_ceiling_mfma_per_wg_iter.argtypes = [ctypes.c_int]
    # Mixes 0-3 and 6: 8 waves; 4 and 5: 4 waves; 32 MFMAs per wave and iteration.
    assert [lib.osc_ceiling_mfma_per_wg_iter(m) for m in range(-1, 8)] == [0, 256, 256, 256, 256, 128, 128, 256, 0]
    invalid = 1  # hipErrorInvalidValue
    for mix, src, out, grid, iters in ((7, BASE, BASE, 1, 1), (-1, BASE, BASE, 1, 1),
                                       (0, None, BASE, 1, 1), (0, BASE, None, 1, 1),
                                       (0, BASE, BASE, 0, 1), (0, BASE, BASE, 1, 0)):
        assert lib.osc_ceiling_launch(mix, src, out, grid, iters, None) == invalid
    lib.osc_lds_read_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    for tr, waves, src, out, grid, iters in ((2, 8, BASE, BASE, 1, 1), (0, 6, BASE, BASE, 1, 1),
                                             (0, 8, None, BASE, 1, 1), (1, 4, BASE, None, 1, 1),
                                             (0, 4, BASE, BASE, 0, 1), (1, 8, BASE, BASE, 1, 0)):
        assert lib.osc_lds_read_launch(tr, waves, src, out, grid, iters, None) == invalid


def test_status_strings():
    for code in osc.STATUS:
        s = osc.attn_status_str(code)
        assert isinstance(s, str) and s
    assert osc.attn_status_str(0) == "ok"
    assert osc.attn_status_str(99) == "unknown status"


def call_attn(q=BASE, k=BASE + 64 * MB, v=BASE + 128 * MB, o=BASE + 192 * MB,
              lse=BASE + 320 * MB, B=1, H=2, N=64, D=128, causal=1, dtype=0):
    lib = osc.load()
    return lib.attn_fwd(q, k, v, o, lse, B, H, N, D, causal, dtype, None)


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_attn_rejects_null(field):
    assert call_attn(**{field: None}) == 1


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(D=0), dict(N=-5),
                                dict(N=1 << 24), dict(B=1 << 40, H=1 << 30),
                                dict(B=1 << 16, H=1 << 15, N=1),          # B*H = 2^31
                                dict(B=1 << 20, H=1 << 4, N=1 << 14)])    # 2^31 workgroups
def test_attn_rejects_bad_shapes(kw):
    assert call_attn(**kw) == 2


@pytest.mark.parametrize("kw", [dict(D=96), dict(D=32), dict(D=256), dict(dtype=2), dict(dtype=-1)])
def test_attn_rejects_unsupported(kw):
    assert call_attn(**kw) == 3


@pytest.mark.parametrize("kw", [dict(q=BASE + 8), dict(k=BASE + 64 * MB + 2),
                                dict(v=BASE + 128 * MB + 4), dict(o=BASE + 192 * MB + 12),
                                dict(lse=BASE + 320 * MB + 2)])
def test_attn_rejects_misaligned(kw):
    assert call_attn(**kw) == 4


@pytest.mark.parametrize("kw", [dict(o=BASE), dict(lse=BASE + 64 * MB + 16),
                                dict(o=BASE + 128 * MB - 64), dict(lse=BASE + 192 * MB + 256)])
def test_attn_rejects_overlap(kw):
    assert call_attn(**kw) == 6


def call_gqa(q=BASE, k=BASE + 64 * MB, v=BASE + 128 * MB, o=BASE + 192 * MB,
             lse=BASE + 320 * MB, B=1, H=8, Hkv=2, N=64, D=128, causal=1, dtype=0):
    return osc.load().attn_fwd_gqa(q, k, v, o, lse, B, H, Hkv, N, D, causal, dtype, None)


@pytest.mark.parametrize("kw", [dict(Hkv=0), dict(Hkv=-2), dict(Hkv=3), dict(Hkv=16),
                                dict(H=6, Hkv=4), dict(H=0, Hkv=1)])
def test_gqa_rejects_bad_head_counts(kw):
    assert call_gqa(**kw) == 2


def test_gqa_other_rejections():
    assert call_gqa(k=None) == 1
    assert call_gqa(D=96) == 3
    assert call_gqa(v=BASE + 128 * MB + 8) == 4
    # K holds B*Hkv = 2 heads of 64x128 fp16 = 32 KiB: an output 16 KiB into K overlaps it.
    assert call_gqa(o=BASE + 64 * MB + 16 * 1024) == 6
    assert call_gqa(lse=BASE + 128 * MB + 32 * 1024 - 4) == 6


def test_splitkv_workspace_sizes():
    """Bytes = segments * B*H*N*(D+2)*4; segments are whole 256-key units."""
    f = osc.attn_fwd_splitkv_workspace
    row = lambda B, H, N, D: B * H * N * (D + 2) * 4
    assert f(1, 2, 16384, 128, 1, 0) == 3 * row(1, 2, 16384, 128)   # few heads: split
    assert f(1, 32, 8192, 128, 1, 0) == 0                            # grid already full
    assert f(1, 4, 256, 128, 1, 0) == 0                              # one 256-key unit
    assert f(1, 8, 4096, 64, 1, 4) == 4 * row(1, 8, 4096, 64)
    assert f(1, 8, 4096, 64, 1, 3) == 3 * row(1, 8, 4096, 64)        # 16 units -> 6,6,4
    assert f(1, 1, 1000, 128, 0, 16) == 4 * row(1, 1, 1000, 128)     # capped by 4 units
    assert f(1, 1, 100, 128, 1, 1) == 0
    assert f(1, 32, 512, 128, 1, 0) == 0                             # short: no split
    assert f(1, 8, 4096, 128, 0, 0) == 2 * row(1, 8, 4096, 128)      # 128 WGs -> 2 segments
    for bad in [(1, 1, 100, 96, 1, 0), (1, 1, 100, 128, 1, 65), (1, 1, 100, 128, 1, -1),
                (0, 1, 100, 128, 1, 0), (1, 1, 0, 128, 1, 0)]:
        assert f(*bad) == -1, bad


WS = BASE + 512 * MB


def call_split(q=BASE, k=BASE + 64 * MB, v=BASE + 128 * MB, o=BASE + 192 * MB,
               lse=BASE + 320 * MB, B=1, H=2, Hkv=2, N=4096, D=128, causal=1, dtype=0,
               splits=4, ws=WS, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = osc.attn_fwd_splitkv_workspace(B, H, N, D, causal, splits)
    return osc.load().attn_fwd_splitkv(q, k, v, o, lse, B, H, Hkv, N, D, causal, dtype, splits,
                                       ws, ws_bytes, None)


def test_splitkv_rejections():
    need = osc.attn_fwd_splitkv_workspace(1, 2, 4096, 128, 1, 4)
    assert need > 0
    assert call_split(splits=65) == 2
    assert call_split(splits=-1) == 2
    assert call_split(Hkv=3) == 2
    assert call_split(D=96) == 3
    assert call_split(ws=None) == 1
    assert call_split(ws=WS + 8) == 4
    assert call_split(ws_bytes=need - 1) == 7
    assert call_split(ws=BASE + 64 * MB + 4096) == 6       # inside K
    assert call_split(ws=BASE + 192 * MB - 256) == 6       # runs into O
    assert call_split(q=None) == 1
    assert osc.attn_status_str(7) != "unknown status"


def test_paged_decode_workspace_sizes():
    """Bytes = segments * B*Hq*(D+2)*4; segments are whole 32-token tiles of
    at most 2048 tokens; the automatic plan aims at about 512 workgroups."""
    f = osc.paged_decode_workspace
    row = lambda B, Hq, D: B * Hq * (D + 2) * 4
    assert f(8, 32, 8, 128, 16, 2048, 0) == 16 * row(8, 32, 128)   # 32K context: 16 x 2048
    assert f(8, 32, 8, 128, 16, 64, 0) == 8 * row(8, 32, 128)      # 1K context: 8 x 128
    assert f(1, 8, 1, 64, 1, 100, 0) == 4 * row(1, 8, 64)          # 4 tiles
    assert f(1, 8, 1, 64, 1, 10, 0) == 0                           # one tile: no split
    assert f(2, 16, 2, 128, 8, 200, 1) == 0                        # one segment requested
    assert f(2, 16, 2, 128, 8, 300, 1) == 2 * row(2, 16, 128)      # 2400 tokens: raised to 2
    assert f(1, 1, 1, 128, 16, 8192, 1) == 64 * row(1, 1, 128)     # 2048-token cap: 64 segments
    assert f(5, 6, 3, 64, 32, 100, 7) == 7 * row(5, 6, 64)
    for bad in [(8, 32, 8, 96, 16, 64, 0), (8, 33, 8, 128, 16, 64, 0), (8, 32, 8, 128, 12, 64, 0),
                (8, 32, 8, 128, 16, 64, -1), (8, 32, 8, 128, 16, 64, 4097), (0, 32, 8, 128, 16, 64, 0),
                (8, 64, 1, 128, 16, 64, 0), (8, 32, 8, 128, 1 << 17, 64, 0),
                (8, 32, 8, 128, 16, 1 << 28, 0)]:
        assert f(*bad) == -1, bad


def call_decode(q=BASE, cache=BASE + 64 * MB, bt=BASE + 8192 * MB, lens=BASE + 8200 * MB,
                o=BASE + 8300 * MB, lse=BASE + 8400 * MB, B=8, Hq=32, Hkv=8, D=128, T=16, P=512,
                max_pages=64, dtype=0, splits=0, ws=BASE + 9000 * MB, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = max(osc.paged_decode_workspace(B, Hq, Hkv, D, T, max_pages, splits), 0)
    return osc.load().paged_decode(q, cache, bt, lens, o, lse, B, Hq, Hkv, D, T, P, max_pages,
                                   dtype, splits, ws, ws_bytes, None)


def test_paged_decode_rejections():
    need = osc.paged_decode_workspace(8, 32, 8, 128, 16, 64, 0)
    assert need > 0
    assert call_decode(q=None) == 1
    assert call_decode(lens=None) == 1
    assert call_decode(ws=None) == 1
    assert call_decode(B=0) == 2
    assert call_decode(Hq=30) == 2
    assert call_decode(splits=-3) == 2
    assert call_decode(B=1 << 16, Hq=1 << 15, Hkv=1 << 15, max_pages=1) == 2   # B*Hq = 2^31
    assert call_decode(P=1 << 31, T=1, Hkv=1, Hq=1, D=64) == 2              # P = 2^31
    assert call_decode(D=80) == 3
    assert call_decode(T=24) == 3
    assert call_decode(Hq=64, Hkv=1) == 3            # group of 64 heads
    assert call_decode(dtype=5) == 3
    assert call_decode(q=BASE + 8) == 4
    assert call_decode(bt=BASE + 8192 * MB + 2) == 4
    assert call_decode(ws=BASE + 9000 * MB + 4) == 4
    assert call_decode(ws_bytes=need - 4) == 7
    assert call_decode(o=BASE + 64 * MB + 4096) == 6   # inside the cache
    assert call_decode(lse=BASE + 8300 * MB + 16) == 6  # inside o
    assert call_decode(ws=BASE + 8200 * MB - 64) == 6   # runs into lengths
    assert call_decode(splits=1, ws=None, ws_bytes=0) != 1  # no workspace needed: not a NULL error


def call_bwd(q=BASE, k=BASE + 64 * MB, v=BASE + 128 * MB, o=BASE + 192 * MB, lse=BASE + 320 * MB,
             do=BASE + 400 * MB, dq=BASE + 500 * MB, dk=BASE + 700 * MB, dv=BASE + 900 * MB,
             B=1, H=2, N=4096, D=128, causal=1, dtype=0, ws=BASE + 1100 * MB, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = max(osc.attn_bwd_workspace(B, H, N), 0)
    return osc.load().attn_bwd(q, k, v, o, lse, do, dq, dk, dv, B, H, N, D, causal, dtype, ws,
                               ws_bytes, None)


def test_attn_bwd_workspace_and_rejections():
    assert osc.attn_bwd_workspace(1, 2, 4096) == 8 * 2 * 4096
    assert osc.attn_bwd_workspace(0, 2, 4096) == -1
    assert call_bwd(do=None) == 1
    assert call_bwd(ws=None) == 1
    assert call_bwd(N=0) == 2
    assert call_bwd(D=96) == 3
    assert call_bwd(dq=BASE + 500 * MB + 8) == 4
    assert call_bwd(ws_bytes=8 * 2 * 4096 - 4) == 7
    assert call_bwd(dk=BASE + 64 * MB) == 6              # dK on top of K
    assert call_bwd(dv=BASE + 700 * MB + 1024) == 6      # dV inside dK
    assert call_bwd(ws=BASE + 192 * MB) == 6             # workspace on O


def call_bwd_gqa(q=BASE, k=BASE + 64 * MB, v=BASE + 128 * MB, o=BASE + 192 * MB,
                 lse=BASE + 320 * MB, do=BASE + 400 * MB, dq=BASE + 500 * MB, dk=BASE + 700 * MB,
                 dv=BASE + 900 * MB, B=1, H=8, Hkv=2, N=4096, D=128, causal=1, dtype=0,
                 ws=BASE + 1100 * MB, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = max(osc.attn_bwd_workspace(B, H, N), 0)
    return osc.load().attn_bwd_gqa(q, k, v, o, lse, do, dq, dk, dv, B, H, Hkv, N, D, causal,
                                   dtype, ws, ws_bytes, None)


def test_attn_bwd_gqa_rejections():
    # Sizes at B1 H8 Hkv2 N4096 D128: q/dO 8 MiB, k/v 2 MiB, dQ 16 MiB, dK/dV 4 MiB.
    assert call_bwd_gqa(k=None) == 1
    assert call_bwd_gqa(Hkv=3) == 2                       # does not divide H
    assert call_bwd_gqa(Hkv=16) == 2                      # more K/V heads than query heads
    assert call_bwd_gqa(Hkv=0) == 2
    assert call_bwd_gqa(dk=BASE + 700 * MB + 4) == 4
    assert call_bwd_gqa(ws_bytes=8 * 8 * 4096 - 4) == 7   # workspace follows the query heads
    assert call_bwd_gqa(dk=BASE + 64 * MB + 2 * MB - 4096) == 6   # dK overlaps the end of K
    assert call_bwd_gqa(dv=BASE + 700 * MB + 4 * MB - 256) == 6   # dV overlaps the end of dK


def test_attn_bwd_is_the_gqa_call_with_one_head_per_group():
    """attn_bwd rejects exactly what attn_bwd_gqa with Hkv = H rejects (every
    case here is invalid, so nothing is launched)."""
    for kw in ({"do": None}, {"N": 0}, {"D": 96}, {"dq": BASE + 500 * MB + 8},
               {"dk": BASE + 64 * MB}, {"ws_bytes": 8 * 2 * 4096 - 4}):
        ref = call_bwd(**kw)
        assert ref != 0
        assert call_bwd_gqa(H=2, Hkv=2, **kw) == ref, kw


def call_softmax(x=BASE, y=BASE + 64 * MB, M=4, N=100):
    return osc.load().row_softmax(x, y, M, N, None)


def test_softmax_rejections():
    assert call_softmax(x=None) == 1
    assert call_softmax(y=None) == 1
    assert call_softmax(M=0) == 2
    assert call_softmax(N=0) == 2
    assert call_softmax(M=1 << 40, N=1 << 30) == 2
    assert call_softmax(M=1 << 31, N=1) == 2      # M < 2^31
    assert call_softmax(M=1, N=1 << 31) == 2      # N < 2^31
    assert call_softmax(x=BASE + 2) == 4
    assert call_softmax(y=BASE + 64 * MB + 1) == 4
    assert call_softmax(y=BASE + 200) == 6


def test_python_binding_raises_with_status():
    with pytest.raises(osc.AttnError) as e:
        osc.attn_fwd(None, BASE, BASE, BASE, BASE, 1, 1, 1, 128, True, "f16", stream=0)
    assert e.value.status == 1
    with pytest.raises(osc.AttnError) as e:
        osc.row_softmax(BASE, BASE + 2 * MB, 1, 0, stream=0)
    assert e.value.status == 2


def test_product_package_never_touches_the_oracle():
    """The HIP path's sources import, link and call nothing under oracle/."""
    pkg = os.path.dirname(osc.__file__)
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if os.path.isfile(path) and path.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
            text = open(path).read()
            assert "oracle" not in text.lower(), path


# The Python binding checks tensor arguments before anything reaches the C
# layer: a CPU tensor would hand the kernel a host address, and a tensor too
# small for the sizes would be written past its end.  These run without a GPU.

def _f16(n):
    import torch
    return torch.zeros(n, dtype=torch.float16)


def _f32(n):
    import torch
    return torch.zeros(n, dtype=torch.float32)


def test_binding_rejects_cpu_tensors():
    B, H, N, D = 1, 2, 8, 64
    n = B * H * N * D
    with pytest.raises(ValueError, match="not on a GPU"):
        osc.attn_fwd(_f16(n), _f16(n), _f16(n), _f32(n), _f32(B * H * N), B, H, N, D, True, "f16", 0)
    with pytest.raises(ValueError, match="not on a GPU"):
        osc.row_softmax(_f32(12), _f32(12), 3, 4, 0)
    import torch
    with pytest.raises(ValueError, match="not on a GPU"):
        osc.attention(torch.zeros((B, H, N, D), dtype=torch.float16),
                      torch.zeros((B, H, N, D), dtype=torch.float16),
                      torch.zeros((B, H, N, D), dtype=torch.float16), True)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_binding_rejects_undersized_tensors(which):
    B, H, N, D = 1, 2, 8, 64
    n = B * H * N * D
    args = {"q": _f16(n), "k": _f16(n), "v": _f16(n), "o": _f32(n), "lse": _f32(B * H * N)}
    short = args[which]
    args[which] = short[: short.numel() - 1]
    with pytest.raises(ValueError, match="elements, the sizes need"):
        osc.attn_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], B, H, N, D, True, "f16", 0)


def test_binding_rejects_wrong_dtypes_and_layouts():
    import torch
    B, H, N, D = 1, 2, 8, 64
    n = B * H * N * D
    with pytest.raises(ValueError, match="must be torch.float32"):
        osc.attn_fwd(_f16(n), _f16(n), _f16(n), _f16(n), _f32(B * H * N), B, H, N, D, True, "f16", 0)
    with pytest.raises(ValueError, match="float16 or bfloat16|dtype says"):
        osc.attn_fwd(_f32(n), _f16(n), _f16(n), _f32(n), _f32(B * H * N), B, H, N, D, True, "f16", 0)
    with pytest.raises(ValueError, match="dtype says"):
        osc.attn_fwd(torch.zeros(n, dtype=torch.bfloat16), torch.zeros(n, dtype=torch.bfloat16),
                     torch.zeros(n, dtype=torch.bfloat16), _f32(n), _f32(B * H * N), B, H, N, D, True,
                     "f16", 0)
    strided = _f32(2 * n)[::2]
    with pytest.raises(ValueError, match="contiguous"):
        osc.attn_fwd(_f16(n), _f16(n), _f16(n), strided, _f32(B * H * N), B, H, N, D, True, "f16", 0)
    with pytest.raises(ValueError, match="int32"):
        osc.paged_decode(_f16(2 * 64), _f16(4 * 2 * 16 * 1 * 64), _f32(2), torch.zeros(1, dtype=torch.int32),
                         _f32(2 * 64), _f32(2), 1, 2, 1, 64, 16, 4, 2, "f16", 0, None, 0, 0)
    with pytest.raises(ValueError, match="bytes, the call needs"):
        osc.attn_fwd_splitkv(_f16(n), _f16(n), _f16(n), _f32(n), _f32(B * H * N), B, H, H, N, D, True,
                             "f16", 2, _f32(3), 16, 0)
    for name, sz in (("dq", n - 1), ("dk", n - 1), ("dv", n - 1)):
        g = {"dq": _f32(n), "dk": _f32(n), "dv": _f32(n)}
        g[name] = _f32(sz)
        with pytest.raises(ValueError, match="elements, the sizes need"):
            osc.attn_bwd(_f16(n), _f16(n), _f16(n), _f32(n), _f32(B * H * N), _f16(n), g["dq"], g["dk"],
                         g["dv"], B, H, N, D, True, "f16", _f32(64), 256, 0)


def test_binding_calls_run_on_the_tensors_device():
    """The binding runs each C call with its tensors' device made current and
    that device's stream: _check reports the common device (None when every
    argument is a raw address, which then runs in the caller's context)."""
    assert osc._check("t", [("a", BASE, "f32", 4), ("b", None, "f32", 4)]) is None
    with osc._on(None):
        pass
