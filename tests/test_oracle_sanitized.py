"""The float64 oracle built with AddressSanitizer, LeakSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only) and driven through every one
of its functions on small, ragged and degenerate inputs with exactly sized
buffers (tests/oracle_sanitize_driver.c): any out-of-bounds access, leak or
undefined operation fails the test.  The oracle is test infrastructure; this
keeps it trustworthy."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_runs_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "sparsekv_oracle.c"),
           os.path.join(HERE, "oracle_sanitize_driver.c"), "-lm", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("the sanitizer runtime is not installed")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stderr[-4000:]
    assert "runtime error" not in run.stderr, run.stderr[-4000:]
    assert "oracle sanitizer run: ok" in run.stdout
