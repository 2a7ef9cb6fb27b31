"""The C-ABI host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the ABI and layer argument tests run in a child process against
libmoe_mi355x_san.so (host code instrumented, device code unchanged) and must
pass with no sanitizer report."""
import os
import subprocess
import sys

import pytest

from sparse_mixture_experts_biased_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_clean_under_asan_and_ubsan(tmp_path):
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("no HIP toolchain to build the sanitized library")
    if B.is_stale(B.SAN_LIB_PATH):
        B.build(sanitize=True)
    env = B.sanitizer_env()
    log = str(tmp_path / "san")
    env["ASAN_OPTIONS"] += f":log_path={log}"
    env["UBSAN_OPTIONS"] += f":log_path={log}"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu",
                          "-p", "no:cacheprovider", "tests/test_abi.py",
                          "tests/test_layer_host.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = [p for p in os.listdir(tmp_path) if p.startswith("san")]
    text = "".join(open(tmp_path / p).read() for p in reports)
    assert res.returncode == 0 and not reports, (res.stdout[-2000:] + res.stderr[-2000:] + text)
    assert "passed" in res.stdout
