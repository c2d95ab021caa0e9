"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer: a gcc build with
-fsanitize=address,undefined (UB aborts) runs the oracle's pin tests in a child process with
gcc's sanitizer runtimes preloaded; the run must pass with no sanitizer report.  (The library's
host code gets the same treatment with selective_state_space_32_amd.build.build_sanitized and
tests/test_abi.py; that build compiles every kernel too and takes minutes, so it is run by hand.)"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    from oracle import oracle
    lib = oracle.build(sanitize=True, out=str(tmp_path / "liboracle_asan.so"))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               LD_PRELOAD=f"{asan}:{ubsan}", SSM_ORACLE_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    print(out[-2000:])
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out
