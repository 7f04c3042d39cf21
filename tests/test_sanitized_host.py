"""The C-ABI host layer (argument validation, launch planning, parameter set-up) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: the ABI tests run against a
copy of the library whose host code carries both sanitizers."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(torch.cuda.is_available(), reason="a CPU-side check")
def test_abi_tests_pass_under_asan_and_ubsan():
    from io_aware_exact_attention_amd.build import asan_runtime, build_sanitized_library
    try:
        lib, rt = build_sanitized_library(), asan_runtime()
    except RuntimeError as e:  # no ROCm toolchain on this host
        pytest.skip(str(e))
    env = dict(os.environ, LD_PRELOAD=rt, MIATTN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
