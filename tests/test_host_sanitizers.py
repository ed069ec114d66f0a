"""The CPU suite under AddressSanitizer and UndefinedBehaviorSanitizer.

The host code of the library (argument validation, the work planner, launch
setup) and the C oracle are built with -fsanitize=address,undefined
(``mla_varlen_prefill_amd.build.build_host_sanitized``,
``oracle.build_sanitized``), and every other CPU test runs against those
builds in a child process with the sanitizer runtime preloaded (the Python
interpreter itself is not instrumented). Any report fails the run. A planted
out-of-bounds read shows that the reports do reach the run in this setup.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from mla_varlen_prefill_amd import build as hip_build  # noqa: E402
import oracle  # noqa: E402

pytestmark = pytest.mark.skipif(not (os.path.exists(hip_build.HIPCC) and os.path.exists(hip_build.CLANGXX)),
                                reason="needs hipcc and clang++")

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


@pytest.fixture(scope="module")
def sanitized():
    lib = hip_build.build_host_sanitized()
    olib = oracle.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=hip_build.asan_runtime(), MLA_PREFILL_LIBRARY=lib, ORACLE_LIBRARY=olib,
               **SAN_ENV)
    return lib, olib, env


def test_sanitized_builds_are_instrumented(sanitized):
    lib, olib, _ = sanitized
    for path in (lib, olib):
        syms = subprocess.run(["nm", "-D", path], check=True, capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, path


def test_cpu_suite_is_clean_under_asan_and_ubsan(sanitized):
    _, _, env = sanitized
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x", "-m", "not gpu",
           "-p", "no:cacheprovider", f"--ignore={os.path.abspath(__file__)}"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out


def test_a_planted_overflow_is_reported(sanitized, tmp_path):
    """A one-element read past a heap array, in code built with the same
    flags, aborts the child with an AddressSanitizer report."""
    _, _, env = sanitized
    src = tmp_path / "planted.c"
    src.write_text(textwrap.dedent("""
        #include <stdlib.h>
        int planted(int n) { int *a = malloc(n * sizeof(int)); for (int i = 0; i < n; ++i) a[i] = i;
                             int s = a[n]; free(a); return s; }
    """))
    so = tmp_path / "libplanted.so"
    clang = shutil.which("clang") or "/opt/rocm/llvm/bin/clang"
    subprocess.run([clang, "-O0", "-g", "-fPIC", "-shared", "-fsanitize=address", "-shared-libasan", str(src), "-o",
                    str(so)], check=True)
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).planted(8)"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
