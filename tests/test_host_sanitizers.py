"""Host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU): the library's host code is built instrumented, and a
driver (tests/host_sanitize/validate.cpp) calls every entry point's argument
validation, each call rejected before any HIP call.  A planted heap overflow
in a separate program built with the same flags checks that the
instrumentation reports."""

import os
import subprocess

import pytest

from binary_coded_precision_amd import build as hb

HERE = os.path.dirname(os.path.abspath(__file__))
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _clang():
    path = os.path.join(os.path.dirname(os.path.realpath(hb.hipcc())), "..", "llvm", "bin",
                        "clang++")
    return path if os.path.exists(path) else "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def driver():
    try:
        return hb.build_host_sanitized(os.path.join(HERE, "host_sanitize", "validate.cpp"))
    except RuntimeError as e:  # a toolchain without the sanitizer runtimes
        pytest.skip("sanitized host build unavailable: %s" % str(e)[:200])


def test_entry_point_validation_is_clean_under_asan_and_ubsan(driver):
    r = subprocess.run([driver], capture_output=True, text=True, timeout=120, env=ENV)
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-2000:]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.strip().endswith("0 failures")


def test_planted_overflow_is_reported(tmp_path, driver):
    src = tmp_path / "overflow.cpp"
    src.write_text("#include <stdlib.h>\n"
                   "int main(int argc, char **argv) {\n"
                   "  volatile int *a = (volatile int *)malloc(4 * sizeof(int));\n"
                   "  a[argc + 3] = 1;  /* one past the end */\n"
                   "  free((void *)a);\n"
                   "  return 0;\n"
                   "}\n")
    exe = tmp_path / "overflow"
    r = subprocess.run([_clang(), "-O1"] + hb.SANITIZE_HOST + [str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60, env=ENV)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
