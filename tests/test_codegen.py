"""Checks on the gfx950 code the compiler makes from the kernel sources (CPU
only: hipcc cross-compiles, nothing runs).

Kernels that issue their buffer-to-LDS loads from inline assembly (the
dma16 / dma4 helpers) write M0 themselves; that is only sound while no
compiler-generated instruction of those files reads or writes M0, which is
checked for every source that calls the helpers.  The kernels must also run
without scratch (register spills) in every instantiation, and the dK/dV loop
must not shuffle its accumulators between registers."""
import os
import re
import shutil
import subprocess

import pytest

from online_softmax_fusion_amd import build as libbuild

needs_hipcc = pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") and not shutil.which("hipcc"),
                                 reason="hipcc not installed")


def device_asm(src, tmp_path):
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    cmd = [libbuild.hipcc(), "--offload-arch=" + libbuild.ARCH, "-O3", "-std=c++17", "-S", "--cuda-device-only",
           os.path.join(libbuild.CSRC, src), "-o", str(out), "-I", os.path.join(libbuild.ROOT, "include"),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + libbuild.EXTRA.get(src, [])
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out.read_text()


def compiler_lines(asm):
    """Instruction lines outside inline-assembly regions."""
    inside = False
    for ln in asm.splitlines():
        if ";;#ASMSTART" in ln:
            inside = True
            continue
        if ";;#ASMEND" in ln:
            inside = False
            continue
        s = ln.strip()
        if not inside and s and not s.startswith(";") and not s.startswith("."):
            yield s


def files_calling_lds_dma():
    """Every kernel source that calls the inline-assembly buffer-to-LDS loads
    (dma16 / dma4 of attn_device.h), which write M0 behind the compiler's back."""
    out = []
    for f in sorted(os.listdir(libbuild.CSRC)):
        if f.endswith(".hip"):
            with open(os.path.join(libbuild.CSRC, f)) as fh:
                if re.search(r"\bdma(?:16|4)\(", fh.read()):
                    out.append(f)
    return out


def test_lds_dma_users_found():
    assert {"decode_bf16.hip", "bwd_bf16.hip"} <= set(files_calling_lds_dma())


@needs_hipcc
@pytest.mark.parametrize("src", files_calling_lds_dma())
def test_m0_only_in_inline_asm(src, tmp_path):
    asm = device_asm(src, tmp_path)
    bad = [s for s in compiler_lines(asm) if re.search(r"\bm0\b", s)]
    assert not bad, bad[:5]
    # and the inline assembly does set it before each buffer-to-LDS load
    assert asm.count("s_mov_b32 m0,") >= asm.count("offen lds") > 0


@needs_hipcc
@pytest.mark.parametrize("src", ["decode_bf16.hip", "prefill_bf16.hip", "bwd_bf16.hip", "l2norm.hip"])
def test_no_scratch(src, tmp_path):
    asm = device_asm(src, tmp_path)
    sizes = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", asm)]
    assert sizes and max(sizes) == 0, sizes


@needs_hipcc
def test_dkdv_loop_keeps_accumulators_in_place(tmp_path):
    """Accumulator-to-accumulator register moves (v_accvgpr_mov) appear in the
    dK/dV kernel only where it zeroes its accumulators (one v_accvgpr_write of
    0, copied to the others), never next to matrix-core work."""
    asm = device_asm("bwd_bf16.hip", tmp_path)
    kernels = list(re.finditer(r"^(_ZN4attn\w*bwd_dkdv_(?:pair_)?kernel\w*):", asm, flags=re.M))
    assert kernels
    for m in kernels:
        body = asm[m.end():asm.index("s_endpgm", m.end())]
        for blk in re.split(r"^\.LBB\d+_\d+:", body, flags=re.M):
            if "v_accvgpr_mov" not in blk:
                continue
            assert "v_mfma" not in blk, m.group(1)
            zero = set()
            for ln in blk.splitlines():
                w = re.search(r"v_accvgpr_write_b32 (a\d+), 0\b", ln)
                if w:
                    zero.add(w.group(1))
                mv = re.search(r"v_accvgpr_mov_b32 (a\d+), (a\d+)", ln)
                if mv:
                    assert mv.group(2) in zero, (m.group(1), ln.strip())   # copies a zero
                    zero.add(mv.group(1))


@needs_hipcc
def test_dq_loop_keeps_accumulators_in_place(tmp_path):
    """The dQ kernel's masked and unmasked tiles share one code path (only the
    elementwise mask branches), so no block with matrix-core work copies
    registers around (a separate masked path made the compiler move the 64
    dQ accumulators after every tile)."""
    asm = device_asm("bwd_bf16.hip", tmp_path)
    kernels = list(re.finditer(r"^(_ZN4attn\w*bwd_dq_kernel\w*):", asm, flags=re.M))
    assert kernels
    for m in kernels:
        body = asm[m.end():asm.index("s_endpgm", m.end())]
        for blk in re.split(r"^\.LBB\d+_\d+:", body, flags=re.M):
            if "v_mfma" in blk:
                moves = len(re.findall(r"\bv_mov_b(?:32|64)\b|v_accvgpr_(?:mov|read|write)", blk))
                assert moves < 8, (m.group(1), moves)
