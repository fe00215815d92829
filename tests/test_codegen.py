"""Checks on the gfx950 code the compiler makes from the kernel sources (CPU
only: hipcc cross-compiles, nothing runs).

The decode kernel issues its buffer-to-LDS loads from inline assembly that
writes M0 itself; that is only sound while no compiler-generated instruction
of that file reads or writes M0.  Both kernels must also run without scratch
(register spills) in every instantiation."""
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


@needs_hipcc
def test_decode_m0_only_in_inline_asm(tmp_path):
    asm = device_asm("decode_bf16.hip", tmp_path)
    bad = [s for s in compiler_lines(asm) if re.search(r"\bm0\b", s)]
    assert not bad, bad[:5]
    # and the inline assembly does set it before each buffer-to-LDS load
    assert asm.count("s_mov_b32 m0,") >= asm.count("offen lds") > 0


@needs_hipcc
@pytest.mark.parametrize("src", ["decode_bf16.hip", "prefill_bf16.hip"])
def test_no_scratch(src, tmp_path):
    asm = device_asm(src, tmp_path)
    sizes = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", asm)]
    assert sizes and max(sizes) == 0, sizes
