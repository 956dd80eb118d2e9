"""The CPU test-suite's oracle pins and boundary tests, run again under AddressSanitizer and
UndefinedBehaviorSanitizer: the oracle (oracle/ga_ref.c) and the library's host code (argument
validation, ga_check_metadata_host, launch planning) built instrumented by
tests/sanitize/build.py, in a Python process that preloads clang's sanitizer runtime.  Any
out-of-bounds access, use after free or undefined behaviour aborts that process."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_oracle_pins_and_boundary_under_sanitizers():
    sys.path.insert(0, os.path.join(ROOT, "tests", "sanitize"))
    import build as san
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": san.runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "GA_ORACLE_LIB": san.build_oracle(),
        "GA_LIBRARY_UNDER_TEST": san.build_library(),
        "OMP_NUM_THREADS": "4",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", "tests/test_oracle_pins.py",
                        "tests/test_boundary.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=850)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
