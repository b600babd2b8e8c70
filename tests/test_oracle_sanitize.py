"""The CPU oracle and the input generator under AddressSanitizer and UndefinedBehaviorSanitizer.

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


def _build_and_run(sources, include, marker):
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "sanitize_run")
        cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
        if include:
            cmd += ["-I", include]
        cmd += sources + ["-lm", "-o", exe]
        build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
            pytest.skip("sanitizer runtime not installed: " + build.stderr[-300:])
        assert build.returncode == 0, build.stderr[-2000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
        assert marker in run.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan():
    _build_and_run([os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "tests", "oracle_sanitize_main.c")],
                   os.path.join(ROOT, "oracle"), "oracle sanitizer run: ok")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_input_generator_under_asan_ubsan():
    """moe_inputs/gen.c (single-threaded here: built without OpenMP) on ragged lengths and the
    storage roundings' edge values."""
    _build_and_run([os.path.join(ROOT, "moe_inputs", "gen.c"),
                    os.path.join(ROOT, "tests", "inputs_sanitize_main.c")],
                   None, "input generator sanitizer run: ok")
