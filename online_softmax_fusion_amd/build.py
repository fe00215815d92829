"""Build ``libattn_mi355x.so`` (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each source is compiled to an object in ``_build/`` (in parallel), then linked
into ``online_softmax_fusion_amd/libattn_mi355x.so``.  Packed-fp32 instruction
selection is switched off for device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn_mi355x.so")
SOURCES = ["prefill_bf16.hip", "decode_bf16.hip", "bwd_bf16.hip", "rows_f32.hip", "combine.hip", "l2norm.hip",
           "noalloc.hip", "attn_api.cpp", "l2norm_api.cpp"]
# per-source device flags: the decode kernel keeps its matrix-core results in
# ordinary VGPRs (its LDS use leaves one workgroup per CU, and the compiler's
# default then moves the accumulators to AGPRs and back on every loop trip)
EXTRA = {"decode_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-c",
           os.path.join(CSRC, src), "-o", obj, "-I", os.path.join(ROOT, "include")]
    if src.endswith(".hip"):
        cmd += ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    cmd += EXTRA.get(src, [])
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(msgs)))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
