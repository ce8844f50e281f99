"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library's sources with the sanitizers on the host side only
(`-Xarch_host`: the gfx950 device code is compiled as usual and never runs
here) together with `tests/abi_host_check.c`, a plain C caller of
include/qlora.h, and runs it with no device visible.  The driver exercises
every validation path, the size helpers at the int64 limits, the codebooks,
the status strings and the timing diagnostics; any sanitizer report (an
out-of-bounds access, a leak, a signed overflow in a size computation) makes
the run fail.  No kernel is launched.
"""

import os
import shutil
import subprocess

import pytest

from nf4_double_quant_amd import build as qbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "abi_host_check.c")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]


def _clang():
    for cand in ("/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout + res.stderr
    return res


def test_abi_host_paths_under_asan_ubsan(tmp_path):
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("host-only check: run where no device is visible")
    try:
        hipcc = qbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    clang = _clang()
    if clang is None:
        pytest.skip("clang not available")
    srcs = [os.path.join(qbuild.CSRC, s) for s in qbuild.SOURCES]
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]
    inc = ["-I", qbuild.INCLUDE, "-I", qbuild.CSRC]
    _run([hipcc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, *inc, "-c", *srcs],
         cwd=tmp_path)
    _run([clang, "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror", *SAN, *inc, "-c", DRIVER,
          "-o", "driver.o"], cwd=tmp_path)
    objs = sorted(str(p) for p in tmp_path.glob("*.o"))
    _run([hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", *objs, "-o", "abi_host_check"], cwd=tmp_path)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(tmp_path / "abi_host_check"), "nodevice"], capture_output=True,
                         text=True, env=env, timeout=120)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert "0 failed" in res.stdout, out
