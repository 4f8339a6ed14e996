"""The oracle's C code under gcc's sanitizers: AddressSanitizer with
UndefinedBehaviorSanitizer (out-of-bounds accesses, leaks, signed overflow,
bad shifts...) and ThreadSanitizer (data races between the row workers).
oracle/sanitize_check.c drives every entry point, threaded and not, and
checks results that follow from the definitions; any sanitizer report makes
the run fail."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRCS = [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "oracle", "sanitize_check.c")]

BUILDS = {
    "asan_ubsan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
    "tsan": ["-fsanitize=thread"],
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
@pytest.mark.parametrize("name", sorted(BUILDS))
def test_oracle_under_sanitizer(name, tmp_path):
    exe = tmp_path / f"oracle_{name}"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-pthread", *BUILDS[name], *SRCS, "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", TSAN_OPTIONS="halt_on_error=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    report = res.stdout + res.stderr
    assert res.returncode == 0, report
    assert "runtime error" not in report and "Sanitizer" not in report, report
    assert "oracle sanitize checks passed" in res.stdout
