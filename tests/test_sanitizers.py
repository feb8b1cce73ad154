"""Host-side sanitizer builds, run on the CPU (no GPU):
  - the CPU oracle (oracle/prism_oracle.c) with gcc's AddressSanitizer and UndefinedBehaviorSanitizer,
    driven through every entry point by tests/sanitize/oracle_driver.c;
  - the C ABI's host side (csrc/prism_api.hip, csrc/prism_prof.hip) with the sanitizers on the host
    pass only, its kernel launchers replaced by the stubs of tests/sanitize/abi_driver.cpp, which
    check that invalid calls return before any launch and that every region carved out of a workspace
    lies inside it.
A sanitizer report, a failed expectation or a non-zero exit fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    rc, log = _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "prism_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
                    "-o", exe, "-lm"])
    assert rc == 0, log
    rc, log = _run([exe], env=ENV)
    assert rc == 0 and "oracle driver ok" in log and "Sanitizer" not in log, log


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_host_side_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    csrc = os.path.join(ROOT, "token_level_sparse_prism_amd", "csrc")
    rc, log = _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    os.path.join(csrc, "prism_api.hip"), os.path.join(csrc, "prism_prof.hip"),
                    os.path.join(SAN, "abi_driver.cpp"), "-o", exe])
    assert rc == 0, log
    rc, log = _run([exe], env=ENV)
    assert rc == 0 and "abi driver ok" in log and "Sanitizer" not in log, log
