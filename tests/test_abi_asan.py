"""The host logic of librlt under AddressSanitizer: argument validation, sizing and the
thread-local error text, exercised by a C++ driver (tests/abi_asan.cpp) linked against every
library source built with host-only ASan. Runs without a GPU."""
import os
import shutil
import subprocess

import pytest

from stateful_decoding_amd import build as rlt_build

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs the ROCm compiler")
def test_host_code_under_address_sanitizer():
    exe = os.path.join(rlt_build.PKG, "_build", "asan", "abi_asan")
    rlt_build.build_host_asan(os.path.join(HERE, "abi_asan.cpp"), exe)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "LeakSanitizer" not in r.stderr
    assert r.stdout.startswith("abi_asan ok"), r.stdout
