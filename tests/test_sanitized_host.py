"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host code (argument checks, host packer, host I2_S paths,
packed-weight files including the fuzzed loader, group plans' validation) and
the oracle are rebuilt with -fsanitize=address,undefined (no recovery), and the
CPU tests that exercise them -- the C-ABI host tests, the binding checks and
every oracle pin -- run again in a child process with the sanitizer runtime
preloaded.  Any out-of-bounds access, use after free or undefined behaviour
aborts that process and fails this test.
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


def test_host_code_under_asan_and_ubsan():
    sys.path.insert(0, str(ROOT))
    from oracle import oracle
    from ternary_weight_bitlinear_amd import build as lib_build

    try:
        runtime = lib_build.asan_runtime()
    except FileNotFoundError:
        pytest.skip("no ASan runtime for the ROCm compiler in this image")
    lib = lib_build.build_sanitized()
    orc = oracle.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=str(runtime), BITNET_LIBRARY=str(lib), BITNET_ORACLE_LIBRARY=str(orc),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           str(ROOT / "tests" / "test_abi_host.py"), str(ROOT / "tests" / "test_binding_host.py"),
           str(ROOT / "tests" / "test_oracle_pins.py")]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr, tail
