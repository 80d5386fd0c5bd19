"""The CPU oracle and the host half of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU needed).

* tests/sanitize/oracle_driver.c runs every oracle entry point (decode,
  full and sampled GEMM, rounding, quantizer over every BF16 pattern,
  argument checks) on exact-size heap buffers, built with gcc;
* tests/sanitize/abi_driver.c runs the library's validation, configuration
  choice, split-K part counts and workspace sizes, built with hipcc for the
  host only (-Xarch_host sanitizers, no device code: an empty offload
  bundle stands in for the kernels, so a call that passes validation stops
  at the device and no kernel can start).
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-o", exe, os.path.join(ROOT, "oracle", "mx_oracle.c"),
          os.path.join(SAN, "oracle_driver.c"), "-lm"])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="4"))
    assert "oracle sanitizer run ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs ROCm hipcc and clang")
def test_abi_host_code_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libmx_asan.so")
    # host code only, sanitized; the device pass is never run
    _run([HIPCC, "--offload-host-only", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-o", lib, os.path.join(ROOT, "block_scaled_precision_mm_amd", "csrc", "mxgemm.hip")])
    # the one symbol the missing device pass would have defined: the offload
    # bundle, here an empty one
    nm = _run(["nm", "-u", lib]).stdout.split()
    sym = next(s for s in nm if s.startswith("__hip_fatbin_"))
    stub = tmp_path / "bundle.c"
    stub.write_text('const char %s[32] __attribute__((aligned(4096))) = "__CLANG_OFFLOAD_BUNDLE__";\n' % sym)
    exe = str(tmp_path / "abi_asan")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe,
          os.path.join(SAN, "abi_driver.c"), str(stub), "-L" + str(tmp_path), "-lmx_asan",
          "-Wl,-rpath," + str(tmp_path), "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert "abi sanitizer run ok" in r.stdout
