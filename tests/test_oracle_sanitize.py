"""The CPU oracle, the input generator and the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer.

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


HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not available")
def test_c_abi_host_code_under_asan_ubsan():
    """The library's host code (argument checks, workspace planning, size queries) built with the
    host sanitizers (its GPU code is built as usual, without them) and driven on the CPU by
    tests/abi_sanitize_main.c: every call fails validation or is a no-op, and the size queries
    are swept to the 32-bit limits."""
    from concurrent.futures import ThreadPoolExecutor
    csrc = os.path.join(ROOT, "bit_expert_ffn_fp32_amd", "csrc")
    sources = sorted(f for f in os.listdir(csrc) if f.endswith(".hip"))
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
                   "-I", os.path.join(ROOT, "include"), "-I", csrc,
                   "-c", os.path.join(csrc, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
            assert r.returncode == 0, r.stderr[-2000:]
            return obj
        with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
            objs = list(ex.map(compile_one, sources))
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
        main_o = os.path.join(tmp, "main.o")
        r = subprocess.run([CLANG, "-std=c11", "-O1", "-g", *san, "-D__HIP_PLATFORM_AMD__",
                            "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                            "-c", os.path.join(ROOT, "tests", "abi_sanitize_main.c"), "-o", main_o],
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        exe = os.path.join(tmp, "abi_sanitize")
        r = subprocess.run([CLANG + "++", *san, main_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                            "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
        assert "C ABI sanitizer run: ok" in run.stdout
