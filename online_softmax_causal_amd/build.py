"""Build libosc_attn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m online_softmax_causal_amd.build

Every HIP source is compiled to an object under ``_build/`` in parallel and
the objects are linked into ``online_softmax_causal_amd/libosc_attn.so``.
``csrc/ceiling.hip``, the matrix-core ceiling probe that ``bench.py
--ceiling`` runs, is linked into its own ``libosc_ceiling.so``: it is
measurement support, not part of the library's interface.
Packed FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libosc_attn.so")
CEILING_LIB = os.path.join(PKG, "libosc_ceiling.so")
SOURCES = ["attn_fwd.hip", "bwd.hip", "decode.hip", "decode_short.hip", "splitkv.hip", "row_softmax.hip",
           "api.hip", "noalloc.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-I" + INCLUDE,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source flags: VGPR-form MFMAs.  In attn_fwd.hip the key-split kernel,
# and in bwd.hip the D = 128 dK/dV kernel, run one wave per SIMD; there the
# compiler would otherwise give the S and dP products AGPR accumulators and
# copy every score out with v_accvgpr_read (one per MFMA in the dK/dV loop).
# The other kernels of attn_fwd.hip compile to the same instructions with or
# without it.  decode_short.hip is the decode kernel built this way, which
# launch_paged_decode uses for short segments only.
SRC_FLAGS = {"attn_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
             "bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
             "decode_short.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + SRC_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, r.stderr))
    return obj


def check_m0(src: str) -> None:
    """The attention, backward and decode kernels write M0 in inline assembly
    (the LDS address of global_load_lds_dword[x4]).  That is only safe while no compiler-generated
    instruction uses M0, so check the generated gfx950 assembly: every M0
    reference must be one of those writes, directly followed by the copy."""
    asm = os.path.join(BUILD, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC] + FLAGS + SRC_FLAGS.get(src, []) + ["-S", "--cuda-device-only",
                                                       os.path.join(CSRC, src), "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc -S failed on %s:\n%s" % (src, r.stderr))
    lines = [ln.split(";")[0].strip() for ln in open(asm)]
    lines = [ln for ln in lines if ln]
    for i, ln in enumerate(lines):
        if "m0" in ln.replace(",", " ").split():
            ok = ln.startswith("s_mov_b32 m0,") and i + 1 < len(lines) and \
                lines[i + 1].startswith("global_load_lds_dword")
            if not ok:
                raise RuntimeError("unexpected use of M0 in %s: %r" % (src, ln))


def _link(objs, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library (and the ceiling
    probe's); returns the library's path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + 3) as ex:
        m0 = [ex.submit(check_m0, src) for src in ("attn_fwd.hip", "decode.hip", "decode_short.hip", "bwd.hip")]
        ceiling = ex.submit(_compile, "ceiling.hip")
        objs = list(ex.map(_compile, SOURCES))
        for f in m0:
            f.result()
        ceiling_obj = ceiling.result()
    _link(objs, LIB)
    _link([ceiling_obj], CEILING_LIB)
    if verbose:
        print("built", LIB)
        print("built", CEILING_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
