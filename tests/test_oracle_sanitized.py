"""The oracle's pins run once more against a build of the oracle with AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): an out-of-bounds access, use after free or undefined arithmetic
anywhere the pins reach aborts the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_converters.py", "tests/test_oracle_router.py", "tests/test_oracle_layer.py",
        "tests/test_oracle_next.py"]


def _asan_runtime():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return os.path.realpath(path) if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_address_and_undefined_behaviour_sanitizers():
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("no ASan runtime for gcc here")
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1", MOE_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PINS], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
