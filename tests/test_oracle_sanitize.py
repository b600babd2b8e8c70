"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_main.c calls every entry point of oracle/oracle.c on small inputs (both code
formats, ragged token counts, k = 1 with one expert, k = E); built here with gcc and
-fsanitize=address,undefined (recovery off), any out-of-bounds access, leak, overflow or other
undefined behaviour in the oracle aborts the program and fails the test.  Host code only: no GPU
code is built with a sanitizer.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitize")
        cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I", os.path.join(ROOT, "oracle"),
               os.path.join(ROOT, "oracle", "oracle.c"),
               os.path.join(ROOT, "tests", "oracle_sanitize_main.c"),
               "-lm", "-o", exe]
        build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
            pytest.skip("sanitizer runtime not installed: " + build.stderr[-300:])
        assert build.returncode == 0, build.stderr[-2000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
        assert "oracle sanitizer run: ok" in run.stdout
