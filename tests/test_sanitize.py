"""The host-side code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU and no HIP runtime involved).

* The argument checks, planners and launch wrappers of the C ABI
  (``attn_api.cpp``, ``l2norm_api.cpp``) are built with g++ together with CPU
  stand-ins for the few HIP runtime calls and for the kernel launchers
  (``tests/sanitize/hip_stubs.cpp``), and driven through every entry point by
  ``tests/sanitize/abi_driver.cpp``: valid calls, invalid arguments, sizes
  far past what the kernels hold, the device topology reaching the kernel
  parameters, and an error left by earlier work not being reported as the
  call's own.
* The fp64 oracle (``oracle/attn_oracle.c``) is built with gcc and run by
  ``tests/sanitize/oracle_driver.c`` over ragged shapes, every mask and bias
  kind, and several threads.

Any sanitizer report aborts the program (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _have(tool):
    return shutil.which(tool) is not None


def _run(cmd, cwd=None):
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=cwd, env=ENV, timeout=600)
    return res.returncode, res.stdout + res.stderr


@pytest.mark.skipif(not _have("g++") or not os.path.isdir("/opt/rocm/include"), reason="g++ or HIP headers missing")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    srcs = [os.path.join(ROOT, p) for p in ("online_softmax_fusion_amd/csrc/attn_api.cpp",
                                              "online_softmax_fusion_amd/csrc/l2norm_api.cpp",
                                              "tests/sanitize/hip_stubs.cpp", "tests/sanitize/abi_driver.cpp")]
    rc, out = _run(["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-o", exe] + srcs)
    assert rc == 0, out
    rc, out = _run([exe])
    assert rc == 0 and "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out
    assert "0 failed" in out, out


@pytest.mark.skipif(not _have("gcc"), reason="gcc missing")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    srcs = [os.path.join(ROOT, "oracle", "attn_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")]
    rc, out = _run(["gcc", "-std=c99"] + SAN + ["-pthread", "-o", exe] + srcs + ["-lm"])
    assert rc == 0, out
    rc, out = _run([exe])
    assert rc == 0 and "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out
    assert "all checks passed" in out, out
