"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:
the fp64 oracle (oracle/gdn_oracle.c: threads, allocation, indexing) driven
by tests/sanitize/oracle_harness.c through exact checks, and the C ABI's
argument checks and workspace sizing (gdn_api.hip, host side only; device
code is compiled but never launched) driven by tests/sanitize/abi_harness.cpp.
A sanitizer report aborts the harness, failing the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_harness")
    _run(["gcc", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-O1", "-g", "-std=c99", os.path.join(ROOT, "oracle", "gdn_oracle.c"),
          os.path.join(HERE, "oracle_harness.c"), "-o", exe, "-lm", "-pthread"], timeout=300)
    r = _run([exe], env=SAN_ENV, timeout=300)
    assert "all checks passed" in r.stdout


def test_abi_argument_checks_under_sanitizers(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_harness")
    csrc = os.path.join(ROOT, "linear_attention_rnn_gdn_amd", "csrc")
    # host-side sanitizers only (each -fsanitize after -Xarch_host); the
    # device code is built as in the library and never launched
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "gdn_api.hip"),
          os.path.join(HERE, "abi_harness.cpp"), "-o", exe], timeout=600)
    r = _run([exe], env=SAN_ENV, timeout=300)
    assert "all checks passed" in r.stdout
